"""Python binding of libmoe, the MI355X (gfx950) mixture-of-experts layer library.

Thin ctypes marshalling over the C ABI declared in ``include/moe.h``: every
function takes torch tensors that already live on the GPU, checks their shape
and dtype, and passes raw device pointers plus the current HIP stream.  All of
the computation runs in the library's HIP kernels; torch only owns memory and
streams.  There is no fallback: if ``libmoe.so`` is missing or fails to load,
importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILES = 0, 1

# names exported by include/moe.h
ABI_FUNCTIONS = ("moe_route", "moe_bucket", "moe_expert_ffn_mxfp4", "moe_ffn_gateup_mxfp4", "moe_ffn_down_mxfp4",
                 "moe_workspace_bytes", "moe_pack_experts", "moe_combine", "moe_layer_mxfp4", "moe_layer_mxfp4_noalloc",
                 "moe_noalloc_scratch_bytes", "moe_cache_create", "moe_cache_destroy",
                 "moe_cache_get_stats", "moe_layer_streamed", "moe_cache_simulate", "q8_0_matmul", "q8_0_matmul_layout", "q8_0_pack", "q8_0_rows",
                 "moe_residual_bf16", "moe_rmsnorm", "moe_argmax_rows", "moe_fnv1a_rows", "moe_mx_mfma_probe",
                 "moe_status_str")


class MoeError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} failed: {_lib.moe_status_str(rc).decode()} (rc={rc})")
        self.rc = rc


class _Experts(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride", ctypes.c_int64), ("d", ctypes.c_int32),
                ("f", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class _CacheConfig(ctypes.Structure):
    _fields_ = [("device_pool", ctypes.c_void_p), ("n_slots", ctypes.c_int32), ("host_pool", ctypes.c_void_p),
                ("n_layers", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d", ctypes.c_int32), ("f", ctypes.c_int32), ("stride", ctypes.c_int64),
                ("n_upload_streams", ctypes.c_int32), ("upload_groups", ctypes.c_int32),
                ("admit_min_rows", ctypes.c_int32), ("n_transient", ctypes.c_int32), ("layout", ctypes.c_int32)]


class _CacheStats(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("admitted", ctypes.c_int64), ("bytes_uploaded", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run router_top_bucket_amd/build.py (or __graft_entry__.build())")
    # torch is imported first, so the HIP runtime torch uses is the one this
    # library binds to (same soname), and torch's streams are valid here
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    EP = ctypes.POINTER(_Experts)
    sigs = {
        "moe_route": (ctypes.c_int, [P, ctypes.c_int, P, P, i32, i32, i32, i32, P, P, P]),
        "moe_bucket": (ctypes.c_int, [P, i32, i32, i32, i32, P, P, P, P, P, P]),
        "moe_expert_ffn_mxfp4": (ctypes.c_int, [P, ctypes.c_int, i32, i32, EP, P, P, P, P, P, P, sz, P]),
        "moe_ffn_gateup_mxfp4": (ctypes.c_int, [P, ctypes.c_int, i32, i32, EP, P, P, P, P, P, sz, P]),
        "moe_ffn_down_mxfp4": (ctypes.c_int, [i32, i32, EP, P, P, P, P, P, P, sz, P]),
        "moe_workspace_bytes": (sz, [i32, i32, EP]),
        "moe_pack_experts": (ctypes.c_int, [P, P, i64, i64, i32, i32, ctypes.c_int, P]),
        "moe_combine": (ctypes.c_int, [P, P, i32, i32, i32, i32, P, P]),
        "moe_layer_mxfp4": (ctypes.c_int, [P, ctypes.c_int, P, P, i32, i32, EP, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "moe_layer_mxfp4_noalloc": (ctypes.c_int, [P, ctypes.c_int, P, P, i32, i32, EP, P, P, P, P, P, P, P, P, P,
                                                   P]),
        "moe_noalloc_scratch_bytes": (sz, []),
        "moe_cache_create": (ctypes.c_int, [ctypes.POINTER(_CacheConfig), ctypes.POINTER(P)]),
        "moe_cache_destroy": (ctypes.c_int, [P]),
        "moe_cache_get_stats": (ctypes.c_int, [P, ctypes.POINTER(_CacheStats)]),
        "moe_layer_streamed": (ctypes.c_int, [P, i32, P, ctypes.c_int, P, P, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                              sz, P]),
        "moe_cache_simulate": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]),
        "q8_0_matmul": (ctypes.c_int, [P, i32, i32, P, P, i32, P, P]),
        "q8_0_matmul_layout": (ctypes.c_int, [P, i32, i32, P, P, i32, P, ctypes.c_int, P]),
        "q8_0_pack": (ctypes.c_int, [P, P, i32, i32, ctypes.c_int, P]),
        "q8_0_rows": (ctypes.c_int, [P, i32, i32, P, P, i32, P, ctypes.c_int, P]),
        "moe_residual_bf16": (ctypes.c_int, [P, P, i64, P, P]),
        "moe_rmsnorm": (ctypes.c_int, [P, i32, i32, ctypes.c_float, P, P, P]),
        "moe_argmax_rows": (ctypes.c_int, [P, i32, i32, P, P]),
        "moe_fnv1a_rows": (ctypes.c_int, [P, i32, i32, P, P]),
        "moe_mx_mfma_probe": (ctypes.c_int, [P, P, P, P, P, P]),
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library_path() -> str:
    return LIB_PATH


def raw_library() -> ctypes.CDLL:
    return _lib


# ----------------------------------------------------------------------------- helpers
def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        return MOE_BF16
    raise ValueError(f"x must be float32 or bfloat16 (got {x.dtype})")


@dataclass
class Experts:
    """One layer's expert records in device memory (see include/moe.h)."""
    base: torch.Tensor  # uint8, (n_routed + n_shared) * stride bytes
    stride: int
    d: int
    f: int
    n_routed: int
    n_shared: int
    whole_layer: bool = True  # False: a descriptor of shapes only (an expert cache's pool)
    layout: int = MOE_LAYOUT_ROWS  # order of the codes planes (moe_pack_experts converts)

    def c_struct(self) -> _Experts:
        if self.base.dtype != torch.uint8:
            raise ValueError("expert base must be a uint8 tensor")
        if self.whole_layer and self.base.numel() < (self.n_routed + self.n_shared) * self.stride:
            raise ValueError("expert base tensor is too small")
        return _Experts(_ptr(self.base), self.stride, self.d, self.f, self.n_routed, self.n_shared, self.layout)


# ----------------------------------------------------------------------------- ABI
def moe_route(x, w_router, logits, k, topk_ids, topk_w, stream=None):
    """Router logits (when w_router is given) then top-k ids and renormalised
    softmax weights.  With w_router None, ``logits`` [M x E] is the input."""
    M, E = logits.shape
    if logits.dtype != torch.float32 or topk_ids.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("logits/topk_w must be float32 and topk_ids int32")
    if tuple(topk_ids.shape) != (M, k) or tuple(topk_w.shape) != (M, k):
        raise ValueError("topk outputs must be [M x k]")
    if w_router is not None:
        if w_router.dtype != torch.float32 or w_router.shape[0] != E or x.shape != (M, w_router.shape[1]):
            raise ValueError("w_router must be float32 [E x d] and x [M x d]")
        d, xdt = w_router.shape[1], _x_dtype(x)
    else:
        d, xdt = 0, (_x_dtype(x) if x is not None else MOE_F32)
    rc = _lib.moe_route(_ptr(x) if w_router is not None else None, xdt, _ptr(w_router), _ptr(logits), M, d, E, k,
                        _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    _check("moe_route", rc)


def moe_bucket(topk_ids, E, n_shared, offsets, perm, active, n_active, dev_error, stream=None):
    """Stable grouping of the M*(k+S) slots by expert."""
    M, k = topk_ids.shape
    for t in (topk_ids, offsets, perm, active, n_active, dev_error):
        if t.dtype != torch.int32:
            raise ValueError("bucket tensors are int32")
    if offsets.numel() < E + n_shared + 1 or perm.numel() < M * (k + n_shared) or active.numel() < E + n_shared:
        raise ValueError("bucket outputs too small")
    rc = _lib.moe_bucket(_ptr(topk_ids), M, k, E, n_shared, _ptr(offsets), _ptr(perm), _ptr(active), _ptr(n_active),
                         _ptr(dev_error), _stream(stream))
    _check("moe_bucket", rc)


def moe_pack_experts(src: torch.Tensor, dst: torch.Tensor, n_records: int, stride: int, d: int, f: int,
                     to_layout: int, stream=None):
    """dst = the n_records records of src with their codes planes in order
    ``to_layout`` (src holds the other order); uint8 tensors on the GPU."""
    for t in (src, dst):
        if t.dtype != torch.uint8 or t.numel() < n_records * stride:
            raise ValueError("src and dst must be uint8 tensors of n_records * stride bytes")
    _check("moe_pack_experts", _lib.moe_pack_experts(_ptr(src), _ptr(dst), n_records, stride, d, f, to_layout,
                                                     _stream(stream)))


def tile_experts(ex: "Experts", stream=None) -> "Experts":
    """A copy of a row-order expert table with its codes planes in tile order."""
    if ex.layout != MOE_LAYOUT_ROWS:
        raise ValueError("expected a row-order expert table")
    n = ex.n_routed + ex.n_shared
    dst = torch.empty(n * ex.stride, dtype=torch.uint8, device=ex.base.device)
    moe_pack_experts(ex.base, dst, n, ex.stride, ex.d, ex.f, MOE_LAYOUT_TILES, stream)
    return Experts(dst, ex.stride, ex.d, ex.f, ex.n_routed, ex.n_shared, layout=MOE_LAYOUT_TILES)


def moe_workspace_bytes(M, k, experts: Experts) -> int:
    s = experts.c_struct()
    return int(_lib.moe_workspace_bytes(M, k, ctypes.byref(s)))


def moe_expert_ffn_mxfp4(x, k, experts: Experts, offsets, perm, active, n_active, y_slots, workspace, stream=None):
    """Every slot's SwiGLU expert output, each expert's weights read once."""
    M = x.shape[0]
    S = experts.n_shared
    if x.shape[1] != experts.d:
        raise ValueError("x must be [M x d]")
    if y_slots.dtype != torch.float32 or tuple(y_slots.shape) != (M * (k + S), experts.d):
        raise ValueError("y_slots must be float32 [M*(k+S) x d]")
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    s = experts.c_struct()
    rc = _lib.moe_expert_ffn_mxfp4(_ptr(x), _x_dtype(x), M, k, ctypes.byref(s), _ptr(offsets), _ptr(perm),
                                   _ptr(active), _ptr(n_active), _ptr(y_slots), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
    _check("moe_expert_ffn_mxfp4", rc)


def moe_ffn_gateup_mxfp4(x, k, experts: Experts, offsets, perm, active, n_active, workspace, stream=None):
    """First FFN stage: h = silu(W_gate x) * (W_up x) per slot, into the workspace."""
    M = x.shape[0]
    if x.shape[1] != experts.d:
        raise ValueError("x must be [M x d]")
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    s = experts.c_struct()
    rc = _lib.moe_ffn_gateup_mxfp4(_ptr(x), _x_dtype(x), M, k, ctypes.byref(s), _ptr(offsets), _ptr(perm),
                                   _ptr(active), _ptr(n_active), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("moe_ffn_gateup_mxfp4", rc)


def moe_ffn_down_mxfp4(M, k, experts: Experts, offsets, perm, active, n_active, y_slots, workspace, stream=None):
    """Second FFN stage: y_slots = W_down h, h read from the workspace the
    gate/up stage filled for the same arguments."""
    S = experts.n_shared
    if y_slots.dtype != torch.float32 or tuple(y_slots.shape) != (M * (k + S), experts.d):
        raise ValueError("y_slots must be float32 [M*(k+S) x d]")
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    s = experts.c_struct()
    rc = _lib.moe_ffn_down_mxfp4(M, k, ctypes.byref(s), _ptr(offsets), _ptr(perm), _ptr(active), _ptr(n_active),
                                 _ptr(y_slots), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("moe_ffn_down_mxfp4", rc)


def moe_combine(y_slots, topk_w, k, n_shared, out, stream=None):
    """out[m] = sum_j w[m,j] y[m,j] + sum_s y_shared[m,s], fp32 in slot order."""
    M, d = out.shape
    if tuple(topk_w.shape) != (M, k) or tuple(y_slots.shape) != (M * (k + n_shared), d):
        raise ValueError("combine shapes")
    rc = _lib.moe_combine(_ptr(y_slots), _ptr(topk_w), M, k, n_shared, d, _ptr(out), _stream(stream))
    _check("moe_combine", rc)


def moe_layer_mxfp4(x, w_router, logits, k, experts: Experts, topk_ids, topk_w, offsets, perm, active, n_active,
                    dev_error, y_slots, out, workspace, stream=None):
    """One layer in one call: what moe_route, moe_bucket, moe_expert_ffn_mxfp4
    and moe_combine give in sequence, bit for bit.  With w_router None,
    ``logits`` [M x E] is the input."""
    M, d = x.shape
    E, S = experts.n_routed, experts.n_shared
    if d != experts.d or tuple(logits.shape) != (M, E) or tuple(out.shape) != (M, d):
        raise ValueError("x [M x d], logits [M x E] and out [M x d] must match the experts")
    if tuple(topk_ids.shape) != (M, k) or tuple(topk_w.shape) != (M, k):
        raise ValueError("topk outputs must be [M x k]")
    if tuple(y_slots.shape) != (M * (k + S), d) or y_slots.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("y_slots must be float32 [M*(k+S) x d], out float32")
    for t in (topk_ids, offsets, perm, active, n_active, dev_error):
        if t.dtype != torch.int32:
            raise ValueError("ids and bucket tensors are int32")
    if offsets.numel() < E + S + 1 or perm.numel() < M * (k + S) or active.numel() < E + S:
        raise ValueError("bucket outputs too small")
    if w_router is not None and (w_router.dtype != torch.float32 or tuple(w_router.shape) != (E, d)):
        raise ValueError("w_router must be float32 [E x d]")
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    s = experts.c_struct()
    rc = _lib.moe_layer_mxfp4(_ptr(x), _x_dtype(x), _ptr(w_router), _ptr(logits), M, k, ctypes.byref(s),
                              _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(perm), _ptr(active), _ptr(n_active),
                              _ptr(dev_error), _ptr(y_slots), _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream(stream))
    _check("moe_layer_mxfp4", rc)


def moe_layer_mxfp4_noalloc(x, w_router, logits, k, experts: Experts, topk_ids, topk_w, offsets, perm, active,
                            n_active, dev_error, y_slots, out, stream=None):
    """moe_layer_mxfp4 with its scratch in the library's static device array
    (no workspace argument; nothing is allocated).  Calls that may overlap on
    one GPU share that array and must be ordered."""
    M, d = x.shape
    E, S = experts.n_routed, experts.n_shared
    if d != experts.d or tuple(logits.shape) != (M, E) or tuple(out.shape) != (M, d):
        raise ValueError("x [M x d], logits [M x E] and out [M x d] must match the experts")
    if tuple(topk_ids.shape) != (M, k) or tuple(topk_w.shape) != (M, k):
        raise ValueError("topk outputs must be [M x k]")
    if tuple(y_slots.shape) != (M * (k + S), d) or y_slots.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("y_slots must be float32 [M*(k+S) x d], out float32")
    for t in (topk_ids, offsets, perm, active, n_active, dev_error):
        if t.dtype != torch.int32:
            raise ValueError("ids and bucket tensors are int32")
    if offsets.numel() < E + S + 1 or perm.numel() < M * (k + S) or active.numel() < E + S:
        raise ValueError("bucket outputs too small")
    if w_router is not None and (w_router.dtype != torch.float32 or tuple(w_router.shape) != (E, d)):
        raise ValueError("w_router must be float32 [E x d]")
    s = experts.c_struct()
    rc = _lib.moe_layer_mxfp4_noalloc(_ptr(x), _x_dtype(x), _ptr(w_router), _ptr(logits), M, k, ctypes.byref(s),
                                      _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(perm), _ptr(active),
                                      _ptr(n_active), _ptr(dev_error), _ptr(y_slots), _ptr(out), _stream(stream))
    _check("moe_layer_mxfp4_noalloc", rc)


def moe_noalloc_scratch_bytes() -> int:
    """Bytes of moe_layer_mxfp4_noalloc's static scratch array."""
    return int(_lib.moe_noalloc_scratch_bytes())


def moe_mx_mfma_probe(a_codes, a_scales, b_codes, b_scales, d, stream=None):
    """One MX-scaled matrix-core instruction: d [16 x 16] fp32 = A x B with
    a_codes [16 x 64] E2M1 bytes, a_scales [16 x 4] E8M0, b_codes [16 x 128]
    E4M3 bytes (column-major B), b_scales [16 x 4] E8M0 (uint8 tensors)."""
    for t, shp in ((a_codes, (16, 64)), (a_scales, (16, 4)), (b_codes, (16, 128)), (b_scales, (16, 4))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"moe_mx_mfma_probe: contiguous uint8 {shp} operands")
    if d.dtype != torch.float32 or tuple(d.shape) != (16, 16) or not d.is_contiguous():
        raise ValueError("moe_mx_mfma_probe: d is a contiguous float32 [16 x 16]")
    _check("moe_mx_mfma_probe", _lib.moe_mx_mfma_probe(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                                                       _ptr(d), _stream(stream)))


def q8_0_pack(src, dst, to_layout, stream=None):
    """dst = the int8 plane src [N x K] in order ``to_layout`` (src in the other order)."""
    N, K = src.shape
    if src.dtype != torch.int8 or dst.dtype != torch.int8 or tuple(dst.shape) != (N, K):
        raise ValueError("q8_0_pack: int8 [N x K] tensors")
    _check("q8_0_pack", _lib.q8_0_pack(_ptr(src), _ptr(dst), N, K, to_layout, _stream(stream)))


def q8_0_matmul(X, Wq, Ws, Y, stream=None, layout=MOE_LAYOUT_ROWS):
    """Y[M x N] = X[M x K] . W^T with W in Q8_0 (int8 [N x K] in order ``layout``,
    fp16 bits [N x K/32])."""
    M, K = X.shape
    N = Wq.shape[0]
    if X.dtype != torch.float32 or Wq.dtype != torch.int8 or Ws.dtype not in (torch.int16, torch.uint16,
                                                                                torch.float16):
        raise ValueError("q8_0 dtypes: X float32, Wq int8, Ws fp16 bits")
    if tuple(Wq.shape) != (N, K) or tuple(Ws.shape) != (N, K // 32) or tuple(Y.shape) != (M, N):
        raise ValueError("q8_0 shapes")
    rc = _lib.q8_0_matmul_layout(_ptr(X), M, K, _ptr(Wq), _ptr(Ws), N, _ptr(Y), layout, _stream(stream))
    _check("q8_0_matmul", rc)


# ----------------------------------------------------------------------------- block-verification helpers
def q8_0_rows(ids, Wq, Ws, X, stream=None, layout=MOE_LAYOUT_ROWS):
    """X[m] = row ids[m] of the Q8_0 matrix (int8 [N x K] in order ``layout``,
    fp16 bits [N x K/32]) in fp32."""
    M, K = X.shape
    N = Wq.shape[0]
    if ids.dtype != torch.int32 or ids.numel() != M or X.dtype != torch.float32 or Wq.dtype != torch.int8:
        raise ValueError("q8_0_rows: ids int32 [M], X float32 [M x K], Wq int8 [N x K]")
    if tuple(Wq.shape) != (N, K) or tuple(Ws.shape) != (N, K // 32):
        raise ValueError("q8_0_rows shapes")
    _check("q8_0_rows", _lib.q8_0_rows(_ptr(ids), M, K, _ptr(Wq), _ptr(Ws), N, _ptr(X), layout, _stream(stream)))


def moe_residual_bf16(h, a=None, h_bf16=None, stream=None):
    """h += a (if given); h_bf16 = bf16(h) rounded to nearest even (if given)."""
    if h.dtype != torch.float32 or (a is not None and (a.dtype != torch.float32 or a.numel() != h.numel())):
        raise ValueError("h and a must be float32 of one size")
    if h_bf16 is not None and (h_bf16.element_size() != 2 or h_bf16.numel() != h.numel()):
        raise ValueError("h_bf16 must hold 16-bit elements, one per h element")
    _check("moe_residual_bf16", _lib.moe_residual_bf16(_ptr(h), _ptr(a), h.numel(), _ptr(h_bf16), _stream(stream)))


def moe_rmsnorm(h, out=None, out_bf16=None, eps=1e-6, stream=None):
    """out / out_bf16 = h / sqrt(mean(h^2) + eps) per row (either may be None, not both)."""
    M, d = h.shape
    if h.dtype != torch.float32 or (out is not None and (out.dtype != torch.float32 or out.shape != h.shape)):
        raise ValueError("h and out must be float32 [M x d]")
    if out_bf16 is not None and (out_bf16.element_size() != 2 or tuple(out_bf16.shape) != (M, d)):
        raise ValueError("out_bf16 must hold 16-bit elements [M x d]")
    _check("moe_rmsnorm", _lib.moe_rmsnorm(_ptr(h), M, d, eps, _ptr(out), _ptr(out_bf16), _stream(stream)))


def moe_argmax_rows(X, idx, stream=None):
    """idx[m] = argmax of row m (lowest index on ties, NaN lowest)."""
    M, N = X.shape
    if X.dtype != torch.float32 or idx.dtype != torch.int32 or idx.numel() < M:
        raise ValueError("X float32 [M x N], idx int32 [M]")
    _check("moe_argmax_rows", _lib.moe_argmax_rows(_ptr(X), M, N, _ptr(idx), _stream(stream)))


def moe_fnv1a_rows(X, hashes, stream=None):
    """hashes[m] = 64-bit FNV-1a of row m's fp32 bytes (an int64 tensor holds the bits)."""
    M, N = X.shape
    if X.dtype != torch.float32 or hashes.dtype != torch.int64 or hashes.numel() < M:
        raise ValueError("X float32 [M x N], hashes int64 [M]")
    _check("moe_fnv1a_rows", _lib.moe_fnv1a_rows(_ptr(X), M, N, _ptr(hashes), _stream(stream)))


# ----------------------------------------------------------------------------- expert streaming
class ExpertCache:
    """A device expert cache in front of a pinned host pool (moe_cache_create).

    ``device_pool``: uint8 GPU tensor of n_slots * stride bytes.  ``host_pool``:
    uint8 PINNED CPU tensor (``pin_memory=True``) of n_layers * (n_routed +
    n_shared) expert records.  Both stay owned by the caller; this object keeps
    references so they outlive the cache."""

    def __init__(self, device_pool: torch.Tensor, host_pool: torch.Tensor, n_layers: int, n_routed: int,
                 n_shared: int, d: int, f: int, stride: int, n_upload_streams: int = 8, upload_groups: int = 4,
                 admit_min_rows: int = 0, n_transient: int = 0, layout: int = MOE_LAYOUT_ROWS):
        if device_pool.dtype != torch.uint8 or not device_pool.is_cuda:
            raise ValueError("device_pool must be a uint8 GPU tensor")
        if host_pool.dtype != torch.uint8 or host_pool.is_cuda or not host_pool.is_pinned():
            raise ValueError("host_pool must be a pinned uint8 CPU tensor")
        if host_pool.numel() < n_layers * (n_routed + n_shared) * stride:
            raise ValueError("host_pool is too small")
        self.device_pool, self.host_pool = device_pool, host_pool
        self.n_slots = device_pool.numel() // stride
        self.n_layers, self.n_routed, self.n_shared, self.d, self.f, self.stride = (n_layers, n_routed, n_shared, d,
                                                                                    f, stride)
        self.layout = layout
        cfg = _CacheConfig(device_pool.data_ptr(), self.n_slots, host_pool.data_ptr(), n_layers, n_routed, n_shared,
                           d, f, stride, n_upload_streams, upload_groups, admit_min_rows, n_transient, layout)
        h = ctypes.c_void_p()
        _check("moe_cache_create", _lib.moe_cache_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h

    def descriptor(self) -> "Experts":
        """An Experts descriptor with this cache's shapes (for buffer sizing;
        the streamed call never addresses records through it)."""
        return Experts(self.device_pool, self.stride, self.d, self.f, self.n_routed, self.n_shared,
                       whole_layer=False, layout=self.layout)

    def stats(self) -> dict:
        st = _CacheStats()
        _check("moe_cache_get_stats", _lib.moe_cache_get_stats(self._h, ctypes.byref(st)))
        return {name: int(getattr(st, name)) for name, _ in _CacheStats._fields_}

    def close(self):
        if self._h:
            _check("moe_cache_destroy", _lib.moe_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_layer_streamed(cache: ExpertCache, layer: int, x, w_router, logits, k, topk_ids, topk_w, offsets, perm,
                       active, n_active, dev_error, y_slots, out, workspace, stream=None):
    """moe_layer_mxfp4 on layer ``layer`` of the cache's host pool, experts
    streamed into the device cache as needed (synchronises the stream once)."""
    M, d = x.shape
    E, S = cache.n_routed, cache.n_shared
    if d != cache.d or tuple(logits.shape) != (M, E) or tuple(out.shape) != (M, d):
        raise ValueError("x [M x d], logits [M x E] and out [M x d] must match the cache")
    if tuple(y_slots.shape) != (M * (k + S), d) or tuple(topk_ids.shape) != (M, k):
        raise ValueError("y_slots [M*(k+S) x d], topk [M x k]")
    rc = _lib.moe_layer_streamed(cache._h, layer, _ptr(x), _x_dtype(x), _ptr(w_router), _ptr(logits), M, k,
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(perm), _ptr(active),
                                 _ptr(n_active), _ptr(dev_error), _ptr(y_slots), _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check("moe_layer_streamed", rc)


def moe_cache_simulate(n_layers, n_routed, n_cache, n_transient, admit_min_rows, calls):
    """Runs the cache policy alone on the host.  ``calls``: list of (layer,
    experts (ascending), rows).  Returns per call (slot, hit, admitted) lists."""
    import numpy as np
    lay = np.array([c[0] for c in calls], dtype=np.int32)
    cn = np.array([len(c[1]) for c in calls], dtype=np.int32)
    ex = np.concatenate([np.asarray(c[1], dtype=np.int32) for c in calls]) if calls else np.zeros(0, np.int32)
    rw = np.concatenate([np.asarray(c[2], dtype=np.int32) for c in calls]) if calls else np.zeros(0, np.int32)
    tot = max(int(cn.sum()), 1)
    slot, hit, adm = (np.zeros(tot, np.int32) for _ in range(3))
    a = lambda v: v.ctypes.data_as(ctypes.c_void_p)
    rc = _lib.moe_cache_simulate(n_layers, n_routed, n_cache, n_transient, admit_min_rows, len(calls), a(lay), a(cn),
                                 a(ex), a(rw), a(slot), a(hit), a(adm))
    _check("moe_cache_simulate", rc)
    out, at = [], 0
    for n in cn:
        out.append((slot[at:at + n].tolist(), hit[at:at + n].tolist(), adm[at:at + n].tolist()))
        at += n
    return out


# ----------------------------------------------------------------------------- one layer
class MoELayer:
    """Buffers for one MoE layer pass over up to ``max_rows`` rows, and the pass
    itself: one moe_layer_mxfp4 call, or (fused=False) the four ABI calls in
    order (route, bucket, expert FFN, combine); both give the same bits."""

    def __init__(self, experts: Experts, k: int, max_rows: int, w_router: torch.Tensor | None = None,
                 device="cuda"):
        self.experts, self.k, self.max_rows, self.w_router = experts, k, max_rows, w_router
        E, S, d = experts.n_routed, experts.n_shared, experts.d
        T = max_rows * (k + S)
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.logits = torch.empty((max_rows, E), **f32)
        self.topk_ids = torch.empty((max_rows, k), **i32)
        self.topk_w = torch.empty((max_rows, k), **f32)
        self.offsets = torch.empty(E + S + 1, **i32)
        self.perm = torch.empty(max(T, 1), **i32)
        self.active = torch.empty(E + S, **i32)
        self.n_active = torch.empty(1, **i32)
        self.dev_error = torch.empty(1, **i32)
        self.y_slots = torch.empty((T, d), **f32)
        self.out = torch.empty((max_rows, d), **f32)
        self.workspace = torch.empty(max(moe_workspace_bytes(max_rows, k, experts), 256), dtype=torch.uint8,
                                     device=device)

    def views(self, M: int):
        S = self.experts.n_shared
        return dict(logits=self.logits[:M], topk_ids=self.topk_ids[:M], topk_w=self.topk_w[:M],
                    offsets=self.offsets, perm=self.perm[:M * (self.k + S)], active=self.active,
                    n_active=self.n_active, dev_error=self.dev_error, y_slots=self.y_slots[:M * (self.k + S)],
                    out=self.out[:M])

    def forward_streamed(self, cache: ExpertCache, layer: int, x: torch.Tensor, logits: torch.Tensor | None = None,
                         stream=None):
        """One layer pass over x [M x d] with layer ``layer`` of the cache's
        host pool (this object must be built on cache.descriptor())."""
        M = x.shape[0]
        if M > self.max_rows:
            raise ValueError("more rows than the layer buffers hold")
        v = self.views(M)
        if logits is not None:
            v["logits"] = logits
        moe_layer_streamed(cache, layer, x, None if logits is not None else self.w_router, v["logits"], self.k,
                           v["topk_ids"], v["topk_w"], v["offsets"], v["perm"], v["active"], v["n_active"],
                           v["dev_error"], v["y_slots"], v["out"], self.workspace, stream)
        return v

    def forward(self, x: torch.Tensor, logits: torch.Tensor | None = None, stream=None, fused: bool = True):
        """One layer pass over x [M x d].  With ``logits`` given the router
        GEMV is skipped and those logits are routed."""
        M = x.shape[0]
        if M > self.max_rows:
            raise ValueError("more rows than the layer buffers hold")
        v = self.views(M)
        E, S = self.experts.n_routed, self.experts.n_shared
        if fused:
            if logits is not None:
                v["logits"] = logits
            moe_layer_mxfp4(x, None if logits is not None else self.w_router, v["logits"], self.k, self.experts,
                            v["topk_ids"], v["topk_w"], v["offsets"], v["perm"], v["active"], v["n_active"],
                            v["dev_error"], v["y_slots"], v["out"], self.workspace, stream)
            return v
        if logits is not None:
            v["logits"] = logits
            moe_route(None, None, logits, self.k, v["topk_ids"], v["topk_w"], stream)
        else:
            moe_route(x, self.w_router, v["logits"], self.k, v["topk_ids"], v["topk_w"], stream)
        moe_bucket(v["topk_ids"], E, S, v["offsets"], v["perm"], v["active"], v["n_active"], v["dev_error"], stream)
        moe_expert_ffn_mxfp4(x, self.k, self.experts, v["offsets"], v["perm"], v["active"], v["n_active"],
                             v["y_slots"], self.workspace, stream)
        moe_combine(v["y_slots"], v["topk_w"], self.k, S, v["out"], stream)
        return v
