"""The FNV-1a reference against the published test vectors of its authors
(the empty string, "a" and "foobar"), and the argmax / bf16 references the
GPU harness tests use, against closed forms."""
import numpy as np

import synth
from oracle.hashes import fnv1a64


def test_fnv1a64_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_fnv1a64_is_order_sensitive_and_bytewise():
    assert fnv1a64(b"ab") != fnv1a64(b"ba")
    x = np.array([1.0, -2.5], dtype=np.float32)
    assert fnv1a64(x.tobytes()) == fnv1a64(bytes(x.view(np.uint8)))


def test_bf16_rne_closed_forms():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0, 1.0 + 2 ** -9], dtype=np.float32)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    assert synth.bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC040, 0x3F80]
