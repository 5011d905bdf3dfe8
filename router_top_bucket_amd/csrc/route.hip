// Router: logits = x . W_r^T, then per row the top-k experts and their
// renormalised softmax weights ("Read the experts the router needs", "Run
// Kimi 3.1 locally on one GPU": the router picks 16 of 896 experts per token).
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ logits
// Workgroup = 256 threads x RW router rows.  Thread th owns the float4 chunks
// th, th+256, ... of the d reduction; its partial sums run over its chunks in
// ascending order, then a fixed butterfly inside each wave and the 4 waves in
// order.  Rows of x are processed 16 at a time; a row's sum never depends on
// how many rows share the launch.
constexpr int LG_RW = 4;
constexpr int LG_THREADS = 256;
constexpr int LG_MCHUNK = 16;
constexpr int LG_KC = 8;  // float4 chunks per thread held in registers per pass

template <int XBF16>
__global__ __launch_bounds__(LG_THREADS) void router_logits_kernel(const void *__restrict__ x,
                                                                   const float *__restrict__ w, int M, int d, int E,
                                                                   float *__restrict__ logits) {
  __shared__ float red[4][LG_RW * LG_MCHUNK];
  const int e0 = blockIdx.x * LG_RW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nchunk = d >> 2;
  for (int mc = 0; mc < M; mc += LG_MCHUNK) {
    const int mn = (M - mc) < LG_MCHUNK ? (M - mc) : LG_MCHUNK;
    float acc[LG_MCHUNK][LG_RW];
#pragma unroll
    for (int m = 0; m < LG_MCHUNK; ++m)
#pragma unroll
      for (int rr = 0; rr < LG_RW; ++rr) acc[m][rr] = 0.f;
    for (int cb = 0; cb < nchunk; cb += LG_THREADS * LG_KC) {
      f32x4 wr[LG_KC][LG_RW];
#pragma unroll
      for (int i = 0; i < LG_KC; ++i) {
        const int c = cb + tid + i * LG_THREADS;
#pragma unroll
        for (int rr = 0; rr < LG_RW; ++rr)
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
          for (int rr = 0; rr < LG_RW; ++rr) {
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
    // fixed-order reduction: butterfly in the wave, then waves 0..3
#pragma unroll
    for (int m = 0; m < LG_MCHUNK; ++m) {
      if (m < mn) {
#pragma unroll
        for (int rr = 0; rr < LG_RW; ++rr) {
          float v = acc[m][rr];
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
          if (lane == 0) red[wv][m * LG_RW + rr] = v;
        }
      }
    }
    __syncthreads();
    if (tid < mn * LG_RW) {
      const int m = tid / LG_RW, rr = tid % LG_RW;
      if (e0 + rr < E) {
        const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        logits[(int64_t)(mc + m) * E + e0 + rr] = v;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ top-k
// One wave per row.  Keys live in LDS; NaN logits rank as -inf and a taken
// entry is marked NaN so it ranks below everything.  Each of k rounds takes
// the wave-wide best by (value desc, index asc) through a butterfly whose
// comparison is a total order, so every lane agrees on the winner.
constexpr int TK_WAVES = 4;

__device__ __forceinline__ bool tk_better(float va, int ia, float vb, int ib) {
  // NaN (taken / empty) is worse than anything
  if (va != va) return false;
  if (vb != vb) return true;
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(TK_WAVES * 64) void topk_kernel(const float *__restrict__ logits, int M, int E, int k,
                                                             int32_t *__restrict__ ids, float *__restrict__ w) {
  extern __shared__ float keys[];  // [TK_WAVES][E]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = blockIdx.x * TK_WAVES + wv;
  if (m >= M) return;  // whole wave exits together; no workgroup barrier below
  float *kr = keys + (int64_t)wv * E;
  const float *row = logits + (int64_t)m * E;
  for (int e = lane; e < E; e += 64) {
    const float v = row[e];
    kr[e] = (v != v) ? -INFINITY : v;
  }
  // key e is only ever written and read by lane e % 64: no cross-lane hazard
  float my_l = 0.f;  // lane j keeps the logit of rank j
  for (int j = 0; j < k; ++j) {
    float bv = __builtin_nanf("");
    int bi = 0x7fffffff;
    for (int e = lane; e < E; e += 64) {
      const float v = kr[e];
      if (tk_better(v, e, bv, bi)) { bv = v; bi = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (tk_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == j) my_l = bv;
    if (lane == 0) ids[(int64_t)m * k + j] = bi;
    if ((bi & 63) == lane && bi < E) kr[bi] = __builtin_nanf("");
  }
  // weights: exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), summed in rank order
  const float l0 = __shfl(my_l, 0, 64);
  const float ej = (lane < k) ? expf(my_l - l0) : 0.f;
  float z = 0.f;
  for (int i = 0; i < k; ++i) z += __shfl(ej, i, 64);
  if (lane < k) w[(int64_t)m * k + lane] = ej / z;
}

// ------------------------------------------------------------------ host
int route_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                 int32_t *ids, float *w, hipStream_t stream) {
  if (w_router) {
    const int grid = (E + LG_RW - 1) / LG_RW;
    if (x_bf16)
      hipLaunchKernelGGL(router_logits_kernel<1>, dim3(grid), dim3(LG_THREADS), 0, stream, x, w_router, M, d, E,
                         logits);
    else
      hipLaunchKernelGGL(router_logits_kernel<0>, dim3(grid), dim3(LG_THREADS), 0, stream, x, w_router, M, d, E,
                         logits);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  const int grid = (M + TK_WAVES - 1) / TK_WAVES;
  hipLaunchKernelGGL(topk_kernel, dim3(grid), dim3(TK_WAVES * 64), (size_t)TK_WAVES * E * sizeof(float), stream,
                     logits, M, E, k, ids, w);
  if (hipGetLastError() != hipSuccess) return -3;
  return 0;
}

}  // namespace moe
