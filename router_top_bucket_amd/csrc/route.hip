// Router: logits = x . W_r^T, then per row the top-k experts and their
// renormalised softmax weights ("Read the experts the router needs", "Run
// Kimi 3.1 locally on one GPU": the router picks 16 of 896 experts per token).
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ logits
// Workgroup = 256 threads x RW router rows.  Thread th owns the float4 chunks
// th, th+256, ... of the d reduction; its partial sums run over its chunks in
// ascending order, then a fixed DPP tree inside each wave and the 4 waves in
// order.  Rows of x are processed 16 at a time.  A logit's arithmetic depends
// only on d (never on M, on RW or on the other rows).
constexpr int LG_THREADS = 256;
constexpr int LG_MCHUNK = 16;
constexpr int LG_KC = 8;  // float4 chunks per thread held in registers per pass

template <int XBF16, int RW>
__global__ __launch_bounds__(LG_THREADS) void router_logits_kernel(const void *__restrict__ x,
                                                                   const float *__restrict__ w, int M, int d, int E,
                                                                   float *__restrict__ logits) {
  __shared__ float red[4][RW * LG_MCHUNK];
  const int e0 = blockIdx.x * RW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nchunk = d >> 2;
  for (int mc = 0; mc < M; mc += LG_MCHUNK) {
    const int mn = (M - mc) < LG_MCHUNK ? (M - mc) : LG_MCHUNK;
    float acc[LG_MCHUNK][RW];
#pragma unroll
    for (int m = 0; m < LG_MCHUNK; ++m)
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) acc[m][rr] = 0.f;
    for (int cb = 0; cb < nchunk; cb += LG_THREADS * LG_KC) {
      f32x4 wr[LG_KC][RW];
#pragma unroll
      for (int i = 0; i < LG_KC; ++i) {
        const int c = cb + tid + i * LG_THREADS;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
          wr[i][rr] = (c < nchunk && e0 + rr < E) ? *(const f32x4 *)(w + (int64_t)(e0 + rr) * d + 4 * c)
                                                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int m = 0; m < LG_MCHUNK; ++m) {
        if (m < mn) {
          const int64_t row = mc + m;
#pragma unroll
          for (int i = 0; i < LG_KC; ++i) {
            const int c = cb + tid + i * LG_THREADS;
            if (c < nchunk) {
              f32x4 xv;
              if (XBF16) {
                const uint2 p = *(const uint2 *)((const uint16_t *)x + row * d + 4 * c);
                xv[0] = __uint_as_float(p.x << 16);
                xv[1] = __uint_as_float(p.x & 0xFFFF0000u);
                xv[2] = __uint_as_float(p.y << 16);
                xv[3] = __uint_as_float(p.y & 0xFFFF0000u);
              } else {
                xv = *(const f32x4 *)((const float *)x + row * d + 4 * c);
              }
#pragma unroll
              for (int rr = 0; rr < RW; ++rr) {
                float a = acc[m][rr];
                a = __builtin_fmaf(wr[i][rr][0], xv[0], a);
                a = __builtin_fmaf(wr[i][rr][1], xv[1], a);
                a = __builtin_fmaf(wr[i][rr][2], xv[2], a);
                a = __builtin_fmaf(wr[i][rr][3], xv[3], a);
                acc[m][rr] = a;
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < LG_MCHUNK; ++m) {
      if (m < mn) {
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
          const float v = wave_sum(acc[m][rr]);
          if (lane == 0) red[wv][m * RW + rr] = v;
        }
      }
    }
    __syncthreads();
    if (tid < mn * RW) {
      const int m = tid / RW, rr = tid % RW;
      if (e0 + rr < E) {
        const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        logits[(int64_t)(mc + m) * E + e0 + rr] = v;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ top-k
// One wave per row, the row's logits in registers (NPL per lane).  Each entry
// becomes a 64-bit key: high word = the logit's bits mapped to an unsigned
// order (NaN as -inf, -0 as +0), low word = ~index, so a larger key is a
// larger logit or, on equal logits, a lower index.  k rounds take the wave
// maximum (a total order: every lane agrees) and retire it.
constexpr int TK_WAVES = 4;

__device__ __forceinline__ uint32_t order_bits(float v) {
  if (v != v) v = -INFINITY;
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int NPL>
__global__ __launch_bounds__(TK_WAVES * 64) void topk_kernel(const float *__restrict__ logits, int M, int E, int k,
                                                             int32_t *__restrict__ ids, float *__restrict__ w) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = blockIdx.x * TK_WAVES + wv;
  if (m >= M) return;  // whole wave; no barrier in this kernel
  const float *row = logits + (int64_t)m * E;
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)order_bits(row[e]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
  }
  float my_l = 0.f;  // lane j keeps the logit of rank j
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
    if (lane == j) my_l = from_order_bits((uint32_t)(best >> 32));
    if (lane == 0) ids[(int64_t)m * k + j] = (int32_t)~(uint32_t)best;
  }
  // weights: exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), summed in rank order
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float ej = (lane < k) ? expf(my_l - l0) : 0.f;
  float z = 0.f;
  for (int i = 0; i < k; ++i) z += __shfl(ej, i, 64);
  if (lane < k) w[(int64_t)m * k + lane] = ej / z;
}

// ------------------------------------------------------------------ host
template <int NPL>
static void launch_topk(const float *logits, int M, int E, int k, int32_t *ids, float *w, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel<NPL>, dim3((M + TK_WAVES - 1) / TK_WAVES), dim3(TK_WAVES * 64), 0, stream, logits,
                     M, E, k, ids, w);
}

template <int XBF16>
static void launch_logits(const void *x, const float *w_router, float *logits, int M, int d, int E,
                          hipStream_t stream) {
  // fewer router rows per workgroup when there are few x rows: more
  // workgroups in flight; the arithmetic of a logit does not change
  if (M <= 4)
    hipLaunchKernelGGL((router_logits_kernel<XBF16, 1>), dim3(E), dim3(LG_THREADS), 0, stream, x, w_router, M, d, E,
                       logits);
  else
    hipLaunchKernelGGL((router_logits_kernel<XBF16, 4>), dim3((E + 3) / 4), dim3(LG_THREADS), 0, stream, x, w_router,
                       M, d, E, logits);
}

int route_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                 int32_t *ids, float *w, hipStream_t stream) {
  if (w_router) {
    if (x_bf16) launch_logits<1>(x, w_router, logits, M, d, E, stream);
    else launch_logits<0>(x, w_router, logits, M, d, E, stream);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  const int npl = (E + 63) / 64;
  if (npl <= 1) launch_topk<1>(logits, M, E, k, ids, w, stream);
  else if (npl <= 2) launch_topk<2>(logits, M, E, k, ids, w, stream);
  else if (npl <= 4) launch_topk<4>(logits, M, E, k, ids, w, stream);
  else if (npl <= 8) launch_topk<8>(logits, M, E, k, ids, w, stream);
  else if (npl <= 14) launch_topk<14>(logits, M, E, k, ids, w, stream);
  else if (npl <= 16) launch_topk<16>(logits, M, E, k, ids, w, stream);
  else if (npl <= 32) launch_topk<32>(logits, M, E, k, ids, w, stream);
  else launch_topk<64>(logits, M, E, k, ids, w, stream);
  if (hipGetLastError() != hipSuccess) return -3;
  return 0;
}

}  // namespace moe
