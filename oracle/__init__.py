"""CPU oracle for the MXFP4 mixture-of-experts layer and the Q8_0 spine matmul.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  The arithmetic
lives in ``oracle.c`` (plain C, one thread per output element); this module
only marshals numpy arrays through ctypes.

Two accumulation readings, chosen per call with ``accum``:
  "f64" (default) every sum in double precision, rounded once when stored;
  "f32" every sum in fp32, a reduction over K as ascending 32-element blocks
        (terms added one by one inside a block, then the block partials in
        order), silu and the softmax with the fp32 expf.
The layer's tolerance is stated against an fp32-accumulating reference; the
fp64 reading is the stricter one (its only rounding is the final store) and
is the one the parity tests use.  A CPU test checks that the two agree far
inside that tolerance at the Kimi shape.

Each function names the passage of "Run Kimi 3.1 locally on one GPU"
(argonautlabs.ai) it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        sig = {
            "orc_max_threads": (ctypes.c_int, []),
            "orc_set_threads": (None, [ctypes.c_int]),
            "orc_e2m1": (ctypes.c_double, [ctypes.c_int]),
            "orc_e8m0": (ctypes.c_double, [ctypes.c_int]),
            "orc_fp16": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_e4m3": (ctypes.c_double, [ctypes.c_int]),
            "orc_mx_tile": (ctypes.c_int, [P, P, P, P, P]),
            "orc_widen_bf16": (None, [P, i64, P]),
            "orc_expert_layout": (ctypes.c_int, [i64, i64, P]),
            "orc_mxfp4_dequant": (ctypes.c_int, [P, P, i64, i64, P]),
            "orc_router_logits": (ctypes.c_int, [P, P, i32, i32, i32, P]),
            "orc_topk": (ctypes.c_int, [P, i32, i32, i32, P, P]),
            "orc_bucket": (ctypes.c_int, [P, i32, i32, i32, i32, P, P, P, P]),
            "orc_expert_ffn": (ctypes.c_int, [P, i32, P, i32, i32, P]),
            "orc_combine": (ctypes.c_int, [P, P, i32, i32, i32, i32, P]),
            "orc_q8_0_matmul": (ctypes.c_int, [P, i32, i32, P, P, i32, P]),
            "orc_router_logits_f32": (ctypes.c_int, [P, P, i32, i32, i32, P]),
            "orc_topk_f32": (ctypes.c_int, [P, i32, i32, i32, P, P]),
            "orc_expert_ffn_f32": (ctypes.c_int, [P, i32, P, i32, i32, P]),
            "orc_combine_f32": (ctypes.c_int, [P, P, i32, i32, i32, i32, P]),
            "orc_q8_0_matmul_f32": (ctypes.c_int, [P, i32, i32, P, P, i32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def _fn(name: str, accum: str):
    """The C function of one step for an accumulation reading."""
    if accum not in ("f64", "f32"):
        raise ValueError(f"accum must be 'f64' or 'f32', not {accum!r}")
    return getattr(_load(), name + ("_f32" if accum == "f32" else ""))


# --------------------------------------------------------------------------- formats
def max_threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads the oracle's later parallel loops use (results do not change)."""
    _load().orc_set_threads(int(n))


def e2m1(code: int) -> float:
    """E2M1 element value (OCP MX v1.0 FP4), as used for the MXFP4 experts."""
    return _load().orc_e2m1(int(code))


def e8m0(b: int) -> float:
    """E8M0 shared scale 2^(b-127); 255 is NaN."""
    return _load().orc_e8m0(int(b))


def e4m3(code: int) -> float:
    """OCP FP8 E4M3 code -> value (NaN for 0x7F / 0xFF)."""
    return float(_load().orc_e4m3(int(code)))


def mx_tile(a_codes: np.ndarray, a_scales: np.ndarray, b_codes: np.ndarray, b_scales: np.ndarray) -> np.ndarray:
    """One MX-scaled 16 x 16 x 128 tile in fp64: A [16 x 64] E2M1 code bytes
    with [16 x 4] E8M0 scales, B given as 16 columns of 128 E4M3 codes with
    [16 x 4] E8M0 scales; returns D [16 x 16] float64."""
    ops = [np.ascontiguousarray(a, dtype=np.uint8) for a in (a_codes, a_scales, b_codes, b_scales)]
    for a, shp in zip(ops, ((16, 64), (16, 4), (16, 128), (16, 4))):
        if a.shape != shp:
            raise ValueError(f"mx_tile: operand of shape {a.shape}, expected {shp}")
    d = np.empty((16, 16), dtype=np.float64)
    _check(_load().orc_mx_tile(*[_ptr(a) for a in ops], _ptr(d)), "mx_tile")
    return d


def fp16(bits: int) -> float:
    """IEEE binary16 bits to a Python float (the Q8_0 block scale)."""
    return _load().orc_fp16(int(bits))


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) widened exactly to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().orc_widen_bf16(_ptr(bits), bits.size, _ptr(out))
    return out


def expert_layout(d: int, f: int) -> list[int]:
    """Byte offsets [gate codes, gate scales, up codes, up scales, down codes,
    down scales, record size] of one expert record."""
    off = np.zeros(7, dtype=np.int64)
    _check(_load().orc_expert_layout(d, f, _ptr(off)), "expert_layout")
    return [int(v) for v in off]


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Dequantise one MXFP4 matrix [rows x K] to float64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    assert codes.size == rows * K // 2 and scales.size == rows * K // 32
    out = np.empty((rows, K), dtype=np.float64)
    _check(_load().orc_mxfp4_dequant(_ptr(codes), _ptr(scales), rows, K, _ptr(out)), "mxfp4_dequant")
    return out


# --------------------------------------------------------------------------- the layer
def as_f32_rows(x: np.ndarray) -> np.ndarray:
    """Rows of x as float32: uint16 arrays are bfloat16 bit patterns."""
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def router_logits(x: np.ndarray, w_r: np.ndarray, accum: str = "f64") -> np.ndarray:
    """logits[M x E] = x[M x d] . W_r[E x d]^T, rounded to fp32 ("Run Kimi 3.1
    locally on one GPU", section "Read the experts the router needs")."""
    xf = as_f32_rows(x)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    M, d = xf.shape
    E = w_r.shape[0]
    out = np.empty((M, E), dtype=np.float32)
    _check(_fn("orc_router_logits", accum)(_ptr(xf), _ptr(w_r), M, d, E, _ptr(out)), "router_logits")
    return out


def topk(logits: np.ndarray, k: int, accum: str = "f64") -> tuple[np.ndarray, np.ndarray]:
    """Top-k expert ids (rank order; ties to the lower index; NaN last) and
    renormalised softmax weights, per row."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = logits.shape
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float32)
    _check(_fn("orc_topk", accum)(_ptr(logits), M, E, k, _ptr(ids), _ptr(w)), "topk")
    return ids, w


def bucket(ids: np.ndarray, E: int, n_shared: int):
    """Stable grouping of slots by expert: (offsets[E+S+1], perm[M*(k+S)],
    active[n_active], n_active)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = ids.shape
    NE = E + n_shared
    offsets = np.empty(NE + 1, dtype=np.int32)
    perm = np.empty(max(M * (k + n_shared), 1), dtype=np.int32)
    active = np.empty(NE, dtype=np.int32)
    na = np.zeros(1, dtype=np.int32)
    _check(_load().orc_bucket(_ptr(ids), M, k, E, n_shared, _ptr(offsets), _ptr(perm), _ptr(active), _ptr(na)),
           "bucket")
    n = int(na[0])
    return offsets, perm[: M * (k + n_shared)], active[:n].copy(), n


def expert_ffn(x_rows: np.ndarray, expert: np.ndarray, d: int, f: int, accum: str = "f64") -> np.ndarray:
    """SwiGLU expert y = W_down (silu(W_gate x) * (W_up x)) for each row of
    x_rows [n x d] (float32 or bfloat16 bits) through one expert record."""
    xf = as_f32_rows(np.atleast_2d(x_rows))
    expert = np.ascontiguousarray(expert, dtype=np.uint8)
    n = xf.shape[0]
    assert xf.shape[1] == d and expert.size >= expert_layout(d, f)[6]
    y = np.empty((n, d), dtype=np.float32)
    _check(_fn("orc_expert_ffn", accum)(_ptr(xf), n, _ptr(expert), d, f, _ptr(y)), "expert_ffn")
    return y


def combine(y_slots: np.ndarray, w: np.ndarray, k: int, n_shared: int, accum: str = "f64") -> np.ndarray:
    """out[m] = sum_j w[m,j] y[m,j] + sum_s y_shared[m,s]."""
    y_slots = np.ascontiguousarray(y_slots, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M = w.shape[0]
    d = y_slots.shape[-1]
    assert y_slots.size == M * (k + n_shared) * d
    out = np.empty((M, d), dtype=np.float32)
    _check(_fn("orc_combine", accum)(_ptr(y_slots), _ptr(w), M, k, n_shared, d, _ptr(out)), "combine")
    return out


def q8_0_matmul(X: np.ndarray, wq: np.ndarray, ws: np.ndarray, accum: str = "f64") -> np.ndarray:
    """Y[M x N] = X[M x K] . W^T with W in Q8_0 (int8 plane, fp16 scale per 32)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    ws = np.ascontiguousarray(ws, dtype=np.uint16)
    M, K = X.shape
    N = wq.shape[0]
    assert wq.shape == (N, K) and ws.shape == (N, K // 32)
    Y = np.empty((M, N), dtype=np.float32)
    _check(_fn("orc_q8_0_matmul", accum)(_ptr(X), M, K, _ptr(wq), _ptr(ws), N, _ptr(Y)), "q8_0_matmul")
    return Y


def layer(x: np.ndarray, k: int, n_routed: int, n_shared: int, d: int, f: int, expert_bytes,
          w_r: np.ndarray | None = None, logits: np.ndarray | None = None, accum: str = "f64"):
    """The whole MoE layer for rows x: router (or given logits) -> top-k ->
    every slot's expert FFN -> combine.  ``expert_bytes(e)`` returns expert e's
    record (shared expert s is e = n_routed + s).  Returns a dict of every
    intermediate the GPU path also produces."""
    xf = as_f32_rows(np.atleast_2d(x))
    M = xf.shape[0]
    if logits is None:
        logits = router_logits(xf, w_r, accum)
    ids, w = topk(logits, k, accum)
    offsets, perm, active, n_active = bucket(ids, n_routed, n_shared)
    S = n_shared
    y_slots = np.zeros((M * (k + S), d), dtype=np.float32)
    for e in active:
        seg = perm[offsets[e]:offsets[e + 1]]
        rows = seg // (k + S)
        y_slots[seg] = expert_ffn(xf[rows], expert_bytes(int(e)), d, f, accum)
    out = combine(y_slots, w, k, S, accum)
    return dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, active=active, n_active=n_active,
                y_slots=y_slots, out=out)
