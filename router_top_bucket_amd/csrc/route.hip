// Router: logits = x . W_r^T, then per row the top-k experts and their
// renormalised softmax weights ("Read the experts the router needs", "Run
// Kimi 3.1 locally on one GPU": the router picks 16 of 896 experts per token).
#include "common.h"
#include "launch.h"

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
// before any arithmetic, so a thread waits for memory once per pass.
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
  typedef typename std::conditional<XBF16 != 0, u32x2, u32x4>::type xraw_t;
  const rsrc_t wres = make_rsrc(w, (uint32_t)((int64_t)E * d * 4));
  const rsrc_t xres = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  for (int mc = 0; mc < M; mc += MCH) {
    const int mn = (M - mc) < MCH ? (M - mc) : MCH;
    float acc[MCH][RW];
#pragma unroll
    for (int m = 0; m < MCH; ++m)
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) acc[m][rr] = 0.f;
    for (int cb = 0; cb < nchunk; cb += LG_THREADS * KC) {
      f32x4 wr[KC][RW];
      xraw_t xr[MCH][KC];
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int c = cb + tid + i * LG_THREADS;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
          wr[i][rr] = __builtin_bit_cast(
              f32x4, buf_load16(wres, (c < nchunk && e0 + rr < E) ? (uint32_t)(((e0 + rr) * d + 4 * c) * 4) : kOOB));
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const uint32_t off = (c < nchunk && m < mn) ? (uint32_t)(((mc + m) * d + 4 * c) * EL) : kOOB;
          if constexpr (XBF16) xr[m][i] = buf_load8(xres, off);
          else xr[m][i] = buf_load16(xres, off);
        }
      }
#pragma unroll
      for (int i = 0; i < KC; ++i) {
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          f32x4 xv;
          if constexpr (XBF16) {
            xv[0] = __uint_as_float(xr[m][i][0] << 16);
            xv[1] = __uint_as_float(xr[m][i][0] & 0xFFFF0000u);
            xv[2] = __uint_as_float(xr[m][i][1] << 16);
            xv[3] = __uint_as_float(xr[m][i][1] & 0xFFFF0000u);
          } else {
            xv = __builtin_bit_cast(f32x4, xr[m][i]);
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

// Batcher's odd-even merge sort of N keys in registers, largest first
// (compile-time network; every index is a constant).
__device__ __forceinline__ void cmpx_desc(uint64_t &a, uint64_t &b) {
  const uint64_t hi = max_u64(a, b), lo = a ^ b ^ hi;
  a = hi;
  b = lo;
}
template <int LO, int HI, int R>  // merge the sorted halves of a[LO..HI] (inclusive), stride R
__device__ __forceinline__ void oem_merge(uint64_t *a) {
  constexpr int STEP = R * 2;
  if constexpr (STEP < HI - LO) {
    oem_merge<LO, HI, STEP>(a);
    oem_merge<LO + R, HI, STEP>(a);
#pragma unroll
    for (int i = LO + R; i < HI - R; i += STEP) cmpx_desc(a[i], a[i + R]);
  } else {
    cmpx_desc(a[LO], a[LO + R]);
  }
}
template <int LO, int HI>  // sort a[LO..HI] (inclusive)
__device__ __forceinline__ void oem_sort(uint64_t *a) {
  if constexpr (HI - LO >= 1) {
    constexpr int MID = LO + (HI - LO) / 2;
    oem_sort<LO, MID>(a);
    oem_sort<MID + 1, HI>(a);
    oem_merge<LO, HI, 1>(a);
  }
}

// Maximum of a 32-bit value over the wave (uniform result): DPP inside each
// 16-lane row, then the four row results.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<MOE_DPP_QUAD_1032>(v));
  v = max(v, dpp_u32<MOE_DPP_QUAD_2301>(v));
  v = max(v, dpp_u32<MOE_DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp_u32<MOE_DPP_ROW_MIRROR>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One wave per row.  Lane l sorts the keys of entries l, l+64, ... largest
// first (P = NPL rounded up to a power of two, padded with key 0, which is
// below every real key) and parks the sorted list in LDS, keeping only its
// head in registers.  Each round takes the largest head over the wave; the
// owning lane (keys are distinct: the index is part of the key) reads its
// next key, and the lane of rank j keeps the round's logit and id.
template <int NPL>
__global__ __launch_bounds__(TK_WAVES * 64) void topk_kernel(const float *__restrict__ logits, int M, int E, int k,
                                                             int32_t *__restrict__ ids, float *__restrict__ w) {
  constexpr int P = NPL <= 1 ? 1 : NPL <= 2 ? 2 : NPL <= 4 ? 4 : NPL <= 8 ? 8 : NPL <= 16 ? 16 : NPL <= 32 ? 32 : 64;
  __shared__ uint64_t lists[TK_WAVES][P + 1][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = blockIdx.x * TK_WAVES + wv;
  if (m >= M) return;  // whole wave; the LDS lists are per wave, no barrier
  const float *row = logits + (int64_t)m * E;
  // all loads first, from a clamped (always valid) index, so none waits on
  // another; entries past E then become key 0
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
  uint64_t key[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = lane + 64 * i;
    key[i] = (i < NPL && e < E) ? (((uint64_t)order_bits(v[i < NPL ? i : 0]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
  }
  oem_sort<0, P - 1>(key);
  uint64_t(*mine)[64] = lists[wv];
#pragma unroll
  for (int i = 1; i < P; ++i) mine[i][lane] = key[i];
  mine[P][lane] = 0ull;  // past the end of every list
  uint64_t head = key[0];
  int pos = 0;  // index of head in this lane's list
  float my_l = 0.f;  // lane j keeps the logit and id of rank j
  int32_t my_id = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = (uint32_t)(head >> 32), lo = (uint32_t)head;
    const uint32_t hmax = wave_max_u32(hi);
    uint64_t cand = __ballot(hi == hmax);
    uint32_t lmax;
    if (__popcll(cand) == 1) {
      lmax = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((unsigned long long)cand) - 1);
    } else {  // equal logits: the lower index (larger ~index) first
      lmax = wave_max_u32(hi == hmax ? lo : 0u);
      cand = __ballot(hi == hmax && lo == lmax);
    }
    if (lane == __ffsll((unsigned long long)cand) - 1) {
      pos = pos < P ? pos + 1 : P;
      head = mine[pos][lane];
    }
    if (lane == j) {
      my_l = from_order_bits(hmax);
      my_id = (int32_t)~lmax;
    }
  }
  if (lane < k) ids[(int64_t)m * k + lane] = my_id;
  // weights: exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), summed in rank order
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float ej = (lane < k) ? expf(my_l - l0) : 0.f;
  float z = 0.f;
  for (int i = 0; i < k; ++i) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ej), i));
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
