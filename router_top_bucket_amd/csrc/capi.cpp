// extern "C" entry points of libmoe: host-side argument validation, then the
// kernels are enqueued on the caller's stream.  Declarations and the contract
// of each function are in include/moe.h.
#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "checks.h"
#include "launch.h"

namespace {

constexpr int kMaxExperts = 4096;  // E + S bound of the single-workgroup bucket and of top-k keys in LDS

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline int status_of(int rc) { return rc == 0 ? MOE_OK : MOE_EHIP; }

inline bool experts_ok(const moe_experts *W) {
  if (!W || !W->base) return false;
  if (W->d <= 0 || W->f <= 0 || W->d % 32 || W->f % 32) return false;
  if (W->n_routed <= 0 || W->n_shared < 0) return false;
  const int64_t rec = (int64_t)3 * W->d * W->f * 17 / 32;
  if (W->stride < rec || W->stride % 16) return false;
  if (reinterpret_cast<uintptr_t>(W->base) % 16) return false;
  if (W->layout != MOE_LAYOUT_ROWS && W->layout != MOE_LAYOUT_TILES) return false;
  return true;
}

// Argument checks shared by the expert-FFN entry points (the full call and
// its two stages).  need_x / need_y say whether that entry point takes x / y.
int ffn_check(const void *x, moe_dtype x_dtype, bool need_x, int32_t M, int32_t k, const moe_experts *W,
              const int32_t *offsets, const int32_t *perm, const int32_t *active, const int32_t *n_active,
              const float *y_slots, bool need_y, const void *workspace, size_t workspace_bytes) {
  if (M < 0 || k < 1 || !experts_ok(W)) return MOE_EINVAL;
  if (need_x) {
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
    if (!x || reinterpret_cast<uintptr_t>(x) % 16) return MOE_EINVAL;
  }
  if (need_y && (!y_slots || reinterpret_cast<uintptr_t>(y_slots) % 16)) return MOE_EINVAL;
  if (!offsets || !perm || !active || !n_active || !workspace) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return MOE_EINVAL;
  if (k > W->n_routed) return MOE_EINVAL;
  if (W->n_routed + W->n_shared > kMaxExperts) return MOE_EUNSUPPORTED;
  if (!moe::ffn_shape_ok(M, k, W->n_shared, W->d, W->f, W->stride)) return MOE_EUNSUPPORTED;
  if ((int64_t)M * (k + W->n_shared) > INT32_MAX / 2) return MOE_EUNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (workspace_bytes < moe::ffn_workspace_bytes(M, k, W->n_shared, W->d, W->f, W->n_routed + W->n_shared))
    return MOE_EINVAL;
  return MOE_OK;
}

int run_ffn(const void *x, moe_dtype x_dtype, int32_t M, int32_t k, const moe_experts *W, const int32_t *offsets,
            const int32_t *perm, const int32_t *active, const int32_t *n_active, float *y_slots, void *workspace,
            int stages, void *stream) {
  return moe::ffn_launch(x, x_dtype == MOE_BF16, M, k, W->base, W->stride, W->d, W->f, W->n_routed, W->n_shared,
                         offsets, perm, active, n_active, y_slots, workspace, stages, nullptr, 0, 0,
                         W->layout == MOE_LAYOUT_TILES, as_stream(stream)) == 0
             ? MOE_OK
             : MOE_EHIP;
}

int route_check(const void *x, moe_dtype x_dtype, const float *w_router, const float *logits, int32_t M, int32_t d,
                int32_t E, int32_t k, const int32_t *topk_ids, const float *topk_w) {
  if (M < 0 || E <= 0 || k < 1 || k > E) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
  if (!logits || !topk_ids || !topk_w) return MOE_EINVAL;
  if (w_router) {
    if (!x || d <= 0 || d % 32) return MOE_EINVAL;
    if (reinterpret_cast<uintptr_t>(w_router) % 16 || reinterpret_cast<uintptr_t>(x) % 16) return MOE_EINVAL;
  }
  if (E > kMaxExperts || k > 64) return MOE_EUNSUPPORTED;
  // router operands are addressed with 32-bit buffer offsets below 2^30
  if (w_router && ((int64_t)E * d * 4 >= (1 << 30) || (int64_t)M * d * 4 >= (1 << 30))) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

}  // namespace

// The argument checks of moe_layer_mxfp4 (also those of moe_layer_streamed).
int moe_layer_check(const void *x, moe_dtype x_dtype, const float *w_router, const float *logits, int32_t M,
                    int32_t k, const moe_experts *W, const int32_t *topk_ids, const float *topk_w,
                    const int32_t *offsets, const int32_t *perm, const int32_t *active, const int32_t *n_active,
                    const int32_t *dev_error, const float *y_slots, const float *out, const void *workspace,
                    size_t workspace_bytes) {
  if (!experts_ok(W)) return MOE_EINVAL;
  const int rc = route_check(x, x_dtype, w_router, logits, M, W->d, W->n_routed, k, topk_ids, topk_w);
  if (rc != MOE_OK) return rc;
  if (!dev_error || !out || reinterpret_cast<uintptr_t>(out) % 16) return MOE_EINVAL;
  return ffn_check(x, x_dtype, true, M, k, W, offsets, perm, active, n_active, y_slots, true, workspace,
                   workspace_bytes);
}

extern "C" {

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: valid but not supported by this build";
    case MOE_EHIP: return "MOE_EHIP: HIP launch or runtime error";
    case MOE_ESCRATCH:
      return "MOE_ESCRATCH: the call needs more scratch than the no-allocation entry point's static array holds";
    default: return "unknown moe_status";
  }
}

int moe_route(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t d,
              int32_t E, int32_t k, int32_t *topk_ids, float *topk_w, void *stream) {
  const int rc = route_check(x, x_dtype, w_router, logits, M, d, E, k, topk_ids, topk_w);
  if (rc != MOE_OK || M == 0) return rc;
  return status_of(moe::route_launch(x, x_dtype == MOE_BF16, w_router, logits, M, d, E, k, topk_ids, topk_w,
                                     as_stream(stream)));
}

int moe_bucket(const int32_t *topk_ids, int32_t M, int32_t k, int32_t E, int32_t n_shared, int32_t *offsets,
               int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error, void *stream) {
  if (M < 0 || k < 1 || E <= 0 || n_shared < 0) return MOE_EINVAL;
  if (!topk_ids || !offsets || !perm || !active || !n_active || !dev_error) return MOE_EINVAL;
  if (E + n_shared > kMaxExperts) return MOE_EUNSUPPORTED;
  if ((int64_t)M * (k + n_shared) > INT32_MAX / 2) return MOE_EUNSUPPORTED;
  if (M == 0) return MOE_OK;
  return status_of(moe::bucket_launch(topk_ids, M, k, E, n_shared, offsets, perm, active, n_active, dev_error,
                                      as_stream(stream)));
}

size_t moe_workspace_bytes(int32_t M, int32_t k, const moe_experts *W) {
  if (M < 0 || k < 1 || !experts_ok(W)) return 0;
  return moe::ffn_workspace_bytes(M, k, W->n_shared, W->d, W->f, W->n_routed + W->n_shared);
}

int moe_expert_ffn_mxfp4(const void *x, moe_dtype x_dtype, int32_t M, int32_t k, const moe_experts *W,
                         const int32_t *offsets, const int32_t *perm, const int32_t *active,
                         const int32_t *n_active, float *y_slots, void *workspace, size_t workspace_bytes,
                         void *stream) {
  const int rc = ffn_check(x, x_dtype, true, M, k, W, offsets, perm, active, n_active, y_slots, true, workspace,
                           workspace_bytes);
  if (rc != MOE_OK || M == 0) return rc;
  return run_ffn(x, x_dtype, M, k, W, offsets, perm, active, n_active, y_slots, workspace,
                 moe::kStageGateUp | moe::kStageDown, stream);
}

int moe_ffn_gateup_mxfp4(const void *x, moe_dtype x_dtype, int32_t M, int32_t k, const moe_experts *W,
                         const int32_t *offsets, const int32_t *perm, const int32_t *active,
                         const int32_t *n_active, void *workspace, size_t workspace_bytes, void *stream) {
  const int rc = ffn_check(x, x_dtype, true, M, k, W, offsets, perm, active, n_active, nullptr, false, workspace,
                           workspace_bytes);
  if (rc != MOE_OK || M == 0) return rc;
  return run_ffn(x, x_dtype, M, k, W, offsets, perm, active, n_active, nullptr, workspace, moe::kStageGateUp,
                 stream);
}

int moe_ffn_down_mxfp4(int32_t M, int32_t k, const moe_experts *W, const int32_t *offsets, const int32_t *perm,
                       const int32_t *active, const int32_t *n_active, float *y_slots, void *workspace,
                       size_t workspace_bytes, void *stream) {
  const int rc = ffn_check(nullptr, MOE_BF16, false, M, k, W, offsets, perm, active, n_active, y_slots, true,
                           workspace, workspace_bytes);
  if (rc != MOE_OK || M == 0) return rc;
  return run_ffn(nullptr, MOE_BF16, M, k, W, offsets, perm, active, n_active, y_slots, workspace, moe::kStageDown,
                 stream);
}

int moe_pack_experts(const uint8_t *src, uint8_t *dst, int64_t n_records, int64_t stride, int32_t d, int32_t f,
                     moe_layout to_layout, void *stream) {
  if (!src || !dst || n_records < 0 || d <= 0 || f <= 0 || d % 32 || f % 32) return MOE_EINVAL;
  if (to_layout != MOE_LAYOUT_ROWS && to_layout != MOE_LAYOUT_TILES) return MOE_EINVAL;
  if (stride < (int64_t)3 * d * f * 17 / 32 || stride % 16) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return MOE_EINVAL;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)(n_records * stride);
  if (a < b + n && b < a + n) return MOE_EINVAL;  // overlapping buffers
  if (n_records == 0) return MOE_OK;
  return status_of(moe::pack_launch(src, dst, n_records, stride, d, f, to_layout == MOE_LAYOUT_TILES,
                                    as_stream(stream)));
}

int moe_combine(const float *y_slots, const float *topk_w, int32_t M, int32_t k, int32_t n_shared, int32_t d,
                float *out, void *stream) {
  if (M < 0 || k < 1 || n_shared < 0 || d <= 0 || d % 4) return MOE_EINVAL;
  if (!y_slots || !topk_w || !out) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(y_slots) % 16 || reinterpret_cast<uintptr_t>(out) % 16) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  return status_of(moe::combine_launch(y_slots, topk_w, M, k, n_shared, d, out, as_stream(stream)));
}

int moe_layer_mxfp4(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t k,
                    const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *perm,
                    int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots, float *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
  const int rc = moe_layer_check(x, x_dtype, w_router, logits, M, k, W, topk_ids, topk_w, offsets, perm, active,
                                 n_active, dev_error, y_slots, out, workspace, workspace_bytes);
  if (rc != MOE_OK || M == 0) return rc;
  return moe_layer_enqueue(x, x_dtype, w_router, logits, M, k, W, topk_ids, topk_w, offsets, perm, active, n_active,
                           dev_error, y_slots, out, workspace, stream);
}

}  // extern "C"

// The kernels of one layer pass (arguments already checked).
int moe_layer_enqueue(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t k,
                      const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *perm,
                      int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots, float *out,
                      void *workspace, void *stream) {
  const int E = W->n_routed, S = W->n_shared, d = W->d;
  const hipStream_t st = as_stream(stream);
  const int bf = x_dtype == MOE_BF16;
  if (moe::ffn_route_fusable(M, bf, d, E, k, S)) {
    // one row: the gate/up launch ranks the logits and writes the routing
    // and bucketing outputs itself (the same code as the top-k and bucket
    // kernels), one launch fewer
    if (w_router && moe::logits_launch(x, bf, w_router, logits, M, d, E, st)) return MOE_EHIP;
    moe::RouteArgs ra;
    ra.logits = logits;
    ra.E = E;
    ra.k = k;
    ra.S = S;
    ra.ids = topk_ids;
    ra.w = topk_w;
    ra.offsets = offsets;
    ra.perm = perm;
    ra.active = active;
    ra.n_active = n_active;
    ra.dev_error = dev_error;
    if (moe::ffn_launch(x, bf, M, k, W->base, W->stride, W->d, W->f, E, S, offsets, perm, active, n_active, y_slots,
                        workspace, moe::kStageGateUp | moe::kStageDown, nullptr, 0, 0,
                        W->layout == MOE_LAYOUT_TILES, st, &ra))
      return MOE_EHIP;
    return status_of(moe::combine_launch(y_slots, topk_w, M, k, S, d, out, st));
  }
  if (moe::route_bucket_launch(x, bf, w_router, logits, M, d, E, k, S, topk_ids, topk_w, offsets, perm, active,
                                n_active, dev_error, st))
    return MOE_EHIP;
  if (run_ffn(x, x_dtype, M, k, W, offsets, perm, active, n_active, y_slots, workspace,
              moe::kStageGateUp | moe::kStageDown, stream) != MOE_OK)
    return MOE_EHIP;
  return status_of(moe::combine_launch(y_slots, topk_w, M, k, S, d, out, st));
}

extern "C" {

int q8_0_matmul_layout(const float *X, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N,
                       float *Y, moe_layout layout, void *stream) {
  if (M < 0 || K <= 0 || K % 32 || N <= 0) return MOE_EINVAL;
  if (!X || !Wq || !Ws || !Y) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(X) % 16 || reinterpret_cast<uintptr_t>(Wq) % 16) return MOE_EINVAL;
  if (layout != MOE_LAYOUT_ROWS && layout != MOE_LAYOUT_TILES) return MOE_EINVAL;
  if (layout == MOE_LAYOUT_TILES && N % 16) return MOE_EINVAL;
  if (M > 8) return MOE_EUNSUPPORTED;
  if ((int64_t)(K / 32 + 2) * 64 * 2 > 65536) return MOE_EUNSUPPORTED;
  if (M == 0) return MOE_OK;
  return status_of(moe::q8_0_launch(X, M, K, Wq, Ws, N, Y, layout == MOE_LAYOUT_TILES, as_stream(stream)));
}

int q8_0_matmul(const float *X, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N, float *Y,
                void *stream) {
  return q8_0_matmul_layout(X, M, K, Wq, Ws, N, Y, MOE_LAYOUT_ROWS, stream);
}

int q8_0_pack(const int8_t *src, int8_t *dst, int32_t N, int32_t K, moe_layout to_layout, void *stream) {
  if (!src || !dst || N <= 0 || K <= 0 || K % 32 || N % 16) return MOE_EINVAL;
  if (to_layout != MOE_LAYOUT_ROWS && to_layout != MOE_LAYOUT_TILES) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return MOE_EINVAL;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)((int64_t)N * K);
  if (a < b + n && b < a + n) return MOE_EINVAL;  // overlapping buffers
  return status_of(moe::q8_0_pack_launch(src, dst, N, K, to_layout == MOE_LAYOUT_TILES, as_stream(stream)));
}

int q8_0_rows(const int32_t *ids, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N, float *X,
              moe_layout layout, void *stream) {
  if (M < 0 || K <= 0 || K % 32 || N <= 0) return MOE_EINVAL;
  if (!ids || !Wq || !Ws || !X) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(X) % 16 || reinterpret_cast<uintptr_t>(Wq) % 4 ||
      reinterpret_cast<uintptr_t>(Ws) % 2)
    return MOE_EINVAL;
  if (layout != MOE_LAYOUT_ROWS && layout != MOE_LAYOUT_TILES) return MOE_EINVAL;
  if (layout == MOE_LAYOUT_TILES && N % 16) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  return status_of(moe::q8_0_rows_launch(ids, M, K, Wq, Ws, N, X, layout == MOE_LAYOUT_TILES, as_stream(stream)));
}

int moe_residual_bf16(float *h, const float *a, int64_t n, uint16_t *h_bf16, void *stream) {
  if (n < 0 || !h || (!a && !h_bf16)) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  return status_of(moe::residual_bf16_launch(h, a, n, h_bf16, as_stream(stream)));
}

int moe_rmsnorm(const float *h, int32_t M, int32_t d, float eps, float *out, uint16_t *out_bf16, void *stream) {
  if (M < 0 || d <= 0 || !h || (!out && !out_bf16) || !(eps >= 0.0f)) return MOE_EINVAL;
  // rows are read and written as float4 / 4 x bf16 when d % 4 == 0
  if (reinterpret_cast<uintptr_t>(h) % 16 || reinterpret_cast<uintptr_t>(out) % 16 ||
      reinterpret_cast<uintptr_t>(out_bf16) % 8)
    return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  return status_of(moe::rmsnorm_launch(h, M, d, eps, out, out_bf16, as_stream(stream)));
}

int moe_argmax_rows(const float *X, int32_t M, int32_t N, int32_t *idx, void *stream) {
  if (M < 0 || N <= 0 || !X || !idx) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(X) % 16) return MOE_EINVAL;  // float4 loads when N % 4 == 0
  if (M == 0) return MOE_OK;
  return status_of(moe::argmax_rows_launch(X, M, N, idx, as_stream(stream)));
}

int moe_fnv1a_rows(const float *X, int32_t M, int32_t N, uint64_t *hash, void *stream) {
  if (M < 0 || N <= 0 || !X || !hash) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(X) % 4 || reinterpret_cast<uintptr_t>(hash) % 8) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  return status_of(moe::fnv1a_rows_launch(X, M, N, hash, as_stream(stream)));
}

}  // extern "C"
