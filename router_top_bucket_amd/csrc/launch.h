// Internal launch interface between the C ABI (capi.cpp) and the kernels.
// Arguments are validated by the caller; these functions only enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

int route_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                 int32_t *ids, float *w, hipStream_t stream);
// the two halves of route_launch: router logits, then top-k + weights
int logits_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E,
                  hipStream_t stream);
int topk_launch(const float *logits, int M, int E, int k, int32_t *ids, float *w, hipStream_t stream);

int bucket_launch(const int32_t *ids, int M, int k, int E, int S, int32_t *offsets, int32_t *perm, int32_t *active,
                  int32_t *n_active, int32_t *dev_error, hipStream_t stream);
// route_launch followed by bucket_launch, with the same results; for up to
// 4 rows the top-k and the bucketing run as one kernel.
int route_bucket_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                        int S, int32_t *ids, float *w, int32_t *offsets, int32_t *perm, int32_t *active,
                        int32_t *n_active, int32_t *dev_error, hipStream_t stream);

// Route mode of the one-row expert FFN: the gate/up launch ranks the logits
// itself and writes the routing and bucketing outputs (ffn_gateup_kernel).
struct RouteArgs {
  const float *logits = nullptr;  // [1 x E]
  int E = 0, k = 0, S = 0;
  int32_t *ids = nullptr;  // [k]
  float *w = nullptr;      // [k]
  int32_t *offsets = nullptr, *perm = nullptr, *active = nullptr, *n_active = nullptr, *dev_error = nullptr;
};
// Whether a layer call of M rows can take route mode.
bool ffn_route_fusable(int64_t M, int x_bf16, int d, int E, int k, int S);

int64_t ffn_max_groups(int64_t M, int k, int S, int n_experts);
size_t ffn_workspace_bytes(int64_t M, int k, int S, int d, int f, int n_experts);
bool ffn_shape_ok(int64_t M, int k, int S, int d, int f, int64_t stride);
// stages: kStageGateUp (group plan + gate/up + SwiGLU into the workspace),
// kStageDown (down projection from the workspace into y), or both.
constexpr int kStageGateUp = 1, kStageDown = 2;
// slot_map (device, [n_routed + n_shared], or null): expert e's record is
// slot_map[e] of the n_records at `experts` (null: record e).  max_active > 0:
// *n_active never exceeds it (sizes the grids with few rows).  tiled: the
// records' codes planes are in tile order (pack_launch).
int ffn_launch(const void *x, int x_bf16, int64_t M, int k, const uint8_t *experts, int64_t stride, int d, int f,
               int n_routed, int n_shared, const int32_t *offsets, const int32_t *perm, const int32_t *active,
               const int32_t *n_active, float *y, void *workspace, int stages, const int32_t *slot_map,
               int n_records, int64_t max_active, int tiled, hipStream_t stream, const RouteArgs *route = nullptr);

// Copies n_records expert records from src to dst (distinct buffers), the
// codes planes permuted from row to tile order (to_tiles) or back; every
// other byte of a record is copied as is.
int pack_launch(const uint8_t *src, uint8_t *dst, int64_t n_records, int64_t stride, int d, int f, int to_tiles,
                hipStream_t stream);

int combine_launch(const float *y, const float *w, int M, int k, int S, int d, float *out, hipStream_t stream);

// tiled: Wq in tile order (N % 16 == 0; q8_0_pack_launch)
int q8_0_launch(const float *X, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *Y, int tiled,
                hipStream_t stream);
int q8_0_pack_launch(const int8_t *src, int8_t *dst, int N, int K, int to_tiles, hipStream_t stream);

// block-verification harness (verify.hip)
int q8_0_rows_launch(const int32_t *ids, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *X,
                     int tiled, hipStream_t stream);
int residual_bf16_launch(float *h, const float *a, int64_t n, uint16_t *hb, hipStream_t stream);
int rmsnorm_launch(const float *h, int M, int d, float eps, float *out, uint16_t *outb, hipStream_t stream);
int argmax_rows_launch(const float *X, int M, int N, int32_t *idx, hipStream_t stream);
int fnv1a_rows_launch(const float *X, int M, int N, uint64_t *hash, hipStream_t stream);

}  // namespace moe
