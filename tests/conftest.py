import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case (full-size oracle work)")


def read_golden(name):
    """Whitespace-separated lines of a golden file, comments dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return num / den if den > 0 else num


def assert_close(got, ref, what="", rel=1e-5, maxabs_frac=1e-4):
    """The layer's floating-point bar: relative L2 error <= 1e-5 and max
    abs error <= 1e-4 * max|ref|, over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    r = rel_l2(got, ref)
    ma = float(np.max(np.abs(got - ref))) if got.size else 0.0
    lim = maxabs_frac * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert r <= rel, f"{what}: rel L2 {r:.3e} > {rel:.1e}"
    assert ma <= lim, f"{what}: max abs {ma:.3e} > {lim:.3e}"
    return r, ma


def make_expert(d, f, gate=(), up=(), down=(), scale_byte=127):
    """Pack an expert record from sparse entries.  Each entry is
    (row, col, code, scale_byte) in the matrix's own [rows x K] indexing:
    gate/up are [f x d], down is [d x f].  Every other code is +0 and every
    other scale byte is ``scale_byte``."""
    mats = []
    for entries, rows, K in ((gate, f, d), (up, f, d), (down, d, f)):
        codes = np.zeros((rows, K // 2), dtype=np.uint8)
        scales = np.full((rows, K // 32), scale_byte, dtype=np.uint8)
        for (r, c, code, sb) in entries:
            b = codes[r, c // 2]
            if c % 2 == 0:
                b = (b & 0xF0) | (code & 15)
            else:
                b = (b & 0x0F) | ((code & 15) << 4)
            codes[r, c // 2] = b
            scales[r, c // 32] = sb
        mats += [codes.ravel(), scales.ravel()]
    return np.concatenate(mats)
