"""64-bit FNV-1a, the logits hash of the pages' run record ("Run Kimi 3.1
locally on one GPU": the block path and plain decoding are compared by their
tokens and by one FNV-1a hash per decoded position's logits).  TEST INFRASTRUCTURE ONLY, like the rest of
``oracle/``.  The definition is Fowler, Noll and Vo's: start from the offset
basis 0xcbf29ce484222325 and for each byte b: h = (h xor b) * 0x100000001b3
modulo 2^64.  Plain Python, one byte at a time."""
from __future__ import annotations

OFFSET_BASIS = 0xCBF29CE484222325
PRIME = 0x100000001B3
MASK = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    h = OFFSET_BASIS
    for b in data:
        h = ((h ^ b) * PRIME) & MASK
    return h
