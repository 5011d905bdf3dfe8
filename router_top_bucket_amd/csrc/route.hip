// Router: logits = x . W_r^T, then per row the top-k experts and their
// renormalised softmax weights ("Run Kimi 3.1 locally on one GPU", section
// "Read the experts the router needs": k = 16 of E = 896 in the Kimi layer).
#include "common.h"
#include "launch.h"
#include "topk.h"

#include <type_traits>

namespace moe {

// ------------------------------------------------------------------ logits
// Workgroup = 256 threads x RW router rows.  Thread th owns the float4 chunks
// th, th+256, ... of the d reduction and accumulates them in ascending order
// (an fma chain per logit), then a fixed DPP tree inside each wave and the 4
// waves in order.  A logit's arithmetic depends only on d: never on M, on RW
// or on the pass shape below.
//
// Rows of x are taken MCH at a time and the reduction KC chunks at a time;
// each pass issues all its loads (W and x, buffer loads: out-of-range chunks
// read zero, and a zero term at the end of a chain leaves it unchanged)
// before any arithmetic; with single-chunk passes (KC = 1) the next pass's
// loads are issued before this pass's arithmetic.
constexpr int LG_THREADS = 256;

template <int XBF16, int RW, int MCH, int KC>
__global__ __launch_bounds__(LG_THREADS) void router_logits_kernel(const void *__restrict__ x,
                                                                   const float *__restrict__ w, int M, int d, int E,
                                                                   float *__restrict__ logits) {
  __shared__ float red[4][RW * MCH];
  const int e0 = blockIdx.x * RW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nchunk = d >> 2;
  constexpr int EL = XBF16 ? 2 : 4;
  constexpr int STEP = LG_THREADS * KC;  // chunks per pass
  typedef typename std::conditional<XBF16 != 0, u32x2, u32x4>::type xraw_t;
  struct Pass {
    f32x4 w[KC][RW];
    xraw_t x[MCH][KC];
  };
  const rsrc_t wres = make_rsrc(w, (uint32_t)((int64_t)E * d * 4));
  const rsrc_t xres = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  for (int mc = 0; mc < M; mc += MCH) {
    const int mn = (M - mc) < MCH ? (M - mc) : MCH;
    float acc[MCH][RW];
#pragma unroll
    for (int m = 0; m < MCH; ++m)
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) acc[m][rr] = 0.f;
    // every load of the pass at chunk base cb (out-of-range chunks read zero)
    auto load = [&](int cb, Pass &ps) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int c = cb + tid + i * LG_THREADS;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
        {
          const uint32_t wo = (c < nchunk && e0 + rr < E) ? (uint32_t)(((e0 + rr) * d + 4 * c) * 4) : kOOB;
          // W is read once when one pass takes every row: stream it
          ps.w[i][rr] = __builtin_bit_cast(f32x4, M <= MCH ? buf_load16_stream(wres, wo) : buf_load16(wres, wo));
        }
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const uint32_t off = (c < nchunk && m < mn) ? (uint32_t)(((mc + m) * d + 4 * c) * EL) : kOOB;
          if constexpr (XBF16) ps.x[m][i] = buf_load8(xres, off);
          else ps.x[m][i] = buf_load16(xres, off);
        }
      }
    };
    auto compute = [&](const Pass &ps) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          f32x4 xv;
          if constexpr (XBF16) {
            xv[0] = __uint_as_float(ps.x[m][i][0] << 16);
            xv[1] = __uint_as_float(ps.x[m][i][0] & 0xFFFF0000u);
            xv[2] = __uint_as_float(ps.x[m][i][1] << 16);
            xv[3] = __uint_as_float(ps.x[m][i][1] & 0xFFFF0000u);
          } else {
            xv = __builtin_bit_cast(f32x4, ps.x[m][i]);
          }
#pragma unroll
          for (int rr = 0; rr < RW; ++rr) {
            float a = acc[m][rr];
            a = __builtin_fmaf(ps.w[i][rr][0], xv[0], a);
            a = __builtin_fmaf(ps.w[i][rr][1], xv[1], a);
            a = __builtin_fmaf(ps.w[i][rr][2], xv[2], a);
            a = __builtin_fmaf(ps.w[i][rr][3], xv[3], a);
            acc[m][rr] = a;
          }
        }
      }
    };
    if (KC > 1 || nchunk <= STEP) {  // one pass at a time
      for (int cb = 0; cb < nchunk; cb += STEP) {
        Pass a;
        load(cb, a);
        compute(a);
      }
    } else {
      // single-chunk passes (the many-row shape): two register sets, so the
      // next pass's loads are in flight while this pass computes (its wait
      // covers only its own, older loads); the chain order of every logit is
      // the same as one pass at a time
      Pass a, b;
      load(0, a);
      for (int cb = 0;;) {
        load(cb + STEP, b);
        compute(a);
        cb += STEP;
        if (cb >= nchunk) break;
        load(cb + STEP, a);
        compute(b);
        cb += STEP;
        if (cb >= nchunk) break;
      }
    }
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
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
// One wave per row (topk_row), TK_WAVES rows per workgroup.
constexpr int TK_WAVES = 4;

template <int NPL>
__global__ __launch_bounds__(TK_WAVES * 64) void topk_kernel(const float *__restrict__ logits, int M, int E, int k,
                                                             int32_t *__restrict__ ids, float *__restrict__ w) {
  constexpr int P = topk_list_len(NPL);
  __shared__ uint64_t lists[TK_WAVES][P + 1][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = blockIdx.x * TK_WAVES + wv;
  if (m >= M) return;  // whole wave; the LDS lists are per wave, no barrier
  int32_t id;
  float wt;
  topk_row<NPL>(logits + (int64_t)m * E, E, k, lists[wv], lane, id, wt);
  if (lane < k) {
    ids[(int64_t)m * k + lane] = id;
    w[(int64_t)m * k + lane] = wt;
  }
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
  // pass shapes by row count (measured on MI355X at E = 896, d = 7168: two
  // router rows per workgroup halve the x re-reads against one and still give
  // 448 workgroups, 2.3x faster than four at 1533 rows); the arithmetic of a
  // logit does not change
  if (M == 1)
    hipLaunchKernelGGL((router_logits_kernel<XBF16, 1, 1, 8>), dim3(E), dim3(LG_THREADS), 0, stream, x, w_router, M,
                       d, E, logits);
  else if (M <= 8)
    hipLaunchKernelGGL((router_logits_kernel<XBF16, 2, 4, 8>), dim3((E + 1) / 2), dim3(LG_THREADS), 0, stream, x,
                       w_router, M, d, E, logits);
  else
    hipLaunchKernelGGL((router_logits_kernel<XBF16, 2, 16, 1>), dim3((E + 1) / 2), dim3(LG_THREADS), 0, stream, x,
                       w_router, M, d, E, logits);
}

int logits_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E,
                  hipStream_t stream) {
  if (x_bf16) launch_logits<1>(x, w_router, logits, M, d, E, stream);
  else launch_logits<0>(x, w_router, logits, M, d, E, stream);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int topk_launch(const float *logits, int M, int E, int k, int32_t *ids, float *w, hipStream_t stream) {
  const int npl = (E + 63) / 64;
  if (npl <= 1) launch_topk<1>(logits, M, E, k, ids, w, stream);
  else if (npl <= 2) launch_topk<2>(logits, M, E, k, ids, w, stream);
  else if (npl <= 4) launch_topk<4>(logits, M, E, k, ids, w, stream);
  else if (npl <= 8) launch_topk<8>(logits, M, E, k, ids, w, stream);
  else if (npl <= 14) launch_topk<14>(logits, M, E, k, ids, w, stream);
  else if (npl <= 16) launch_topk<16>(logits, M, E, k, ids, w, stream);
  else if (npl <= 32) launch_topk<32>(logits, M, E, k, ids, w, stream);
  else launch_topk<64>(logits, M, E, k, ids, w, stream);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int route_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                 int32_t *ids, float *w, hipStream_t stream) {
  if (w_router && logits_launch(x, x_bf16, w_router, logits, M, d, E, stream)) return -3;
  return topk_launch(logits, M, E, k, ids, w, stream);
}

}  // namespace moe
