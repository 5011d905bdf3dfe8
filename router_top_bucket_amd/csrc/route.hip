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
// loads are issued before this pass's arithmetic.  With XS > 1 the
// workgroup holds XS such 256-thread sets over the same router rows, set s
// taking x rows s*MCH.. of each XS*MCH (more independent waves per router
// row, each with a shorter list of rows; every logit's chain is unchanged).
constexpr int LG_THREADS = 256;

template <int XBF16, int RW, int MCH, int KC, int XS = 1>
__global__ __launch_bounds__(LG_THREADS * XS) void router_logits_kernel(const void *__restrict__ x,
                                                                        const float *__restrict__ w, int M, int d,
                                                                        int E, float *__restrict__ logits) {
  __shared__ float reds[XS][4][RW * MCH];
  const int e0 = blockIdx.x * RW;
  const int xs = threadIdx.x / LG_THREADS;
  const int tid = threadIdx.x % LG_THREADS, lane = tid & 63, wv = tid >> 6;
  float (&red)[4][RW * MCH] = reds[xs];
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
  // every set takes the same trip count (the barriers below are the
  // workgroup's); a set past the last row loads zeros and stores nothing
  for (int mc0 = 0; mc0 < M; mc0 += MCH * XS) {
    const int mc = mc0 + xs * MCH;
    const int mn = (M - mc) < MCH ? ((M - mc) > 0 ? (M - mc) : 0) : MCH;
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
          // W is read once when one pass of one set takes every row: stream it
          ps.w[i][rr] =
              __builtin_bit_cast(f32x4, XS == 1 && M <= MCH ? buf_load16_stream(wres, wo) : buf_load16(wres, wo));
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

// ------------------------------------------------------------------ logits on MFMA (more than 16 rows)
// logits[m, e] = sum_c W_r[e, c] x[m, c] on bf16 MFMA with fp32 accumulation
// and exact products: every fp32 weight is split exactly into three bf16
// parts (split3_x8), bf16 x is used as is and fp32 x is split into three
// parts as well.  The reduction over d is cut into slices of 32 elements;
// slice c belongs to range q = c mod 16.  Range q's partial sum P_q is one
// MFMA accumulator chain over its slices in ascending order, each slice
// adding W_hi, W_mid, W_lo times each x part in the order (x part, W part).
// The logit is ((P_0 + P_1) + P_2) + ... + P_15 in fp32.  That arithmetic
// depends on d alone: the rows of one call do not influence each other (an
// MFMA output element depends only on its own A row, B column and
// accumulator).  Calls of up to 16 rows use the VALU form above, whose
// summation order differs: a row's logits agree across the two forms within
// rounding, not bit for bit (prefill rows are compared within tolerance).
// Workgroup = one wave: 16 TR router rows x 16 TX x rows.  The ranges run
// one after another (each chain is the same sequence of MFMAs as with all
// ranges interleaved), so a tile needs only the running chain and the sum
// of the finished ranges; per slice TR A fragments (W, three parts) and TX B
// fragments, a ring of NR slices in flight.
constexpr int kRqRanges = 16;
constexpr int kRqMaxRows = 16;  // calls of up to this many rows take the VALU form

// Three bf16 parts of 8 fp32 values, v == hi + mid + lo exactly: hi is v
// truncated to its top 16 bits, r = v - hi is exact, mid is r truncated and
// lo = r - mid is exact and has at most 8 significant bits (v has 24), so it
// is a bf16 value.  A part's bf16 is the top half of its fp32 bits.
__device__ __forceinline__ void split3_x8(const float (&v)[8], bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
  u32x4 h, m, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t u = __float_as_uint(v[2 * e + t]);
      hb[t] = u & 0xFFFF0000u;
      const float r = v[2 * e + t] - __uint_as_float(hb[t]);
      mb[t] = __float_as_uint(r) & 0xFFFF0000u;
      lb[t] = __float_as_uint(r - __uint_as_float(mb[t]));
    }
    // high halves of two fp32 words -> one dword of two bf16 (element 2e low)
    h[e] = __builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u);
    m[e] = __builtin_amdgcn_perm(mb[1], mb[0], 0x07060302u);
    l[e] = __builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u);
  }
  hi = bits_to_bf16x8(h);
  mid = bits_to_bf16x8(m);
  lo = bits_to_bf16x8(l);
}

// The x parts' order in a chain, then the W parts' (both forms).
template <int NP>
__device__ __forceinline__ f32x4 rq_chain(const bf16x8 (&a)[3], const bf16x8 (&b)[NP], f32x4 acc) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int w = 0; w < 3; ++w) acc = mfma16x16x32(a[w], b[p], acc);
  return acc;
}

template <int XBF16, int NR, int TR, int TX>
__global__ __launch_bounds__(64) void router_mfma_tile_kernel(const void *__restrict__ x, const float *__restrict__ w,
                                                              int M, int d, int E, float *__restrict__ logits) {
  constexpr int NP = XBF16 ? 1 : 3;
  constexpr int EL = XBF16 ? 2 : 4;
  static_assert(kRqRanges % NR == 0, "the ring depth divides a range round");
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, kg = lane >> 4;
  const int e0 = blockIdx.x * 16 * TR, m0 = blockIdx.y * 16 * TX;
  const int nsl = d / 32;
  const int nper = (nsl + kRqRanges - 1) / kRqRanges;  // slices per range, the last ones past d are zeros
  const int total = kRqRanges * nper;
  const rsrc_t wres = make_rsrc(w, (uint32_t)((int64_t)E * d * 4));
  const rsrc_t xres = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  uint32_t wbase[TR], xbase[TX];
#pragma unroll
  for (int tr = 0; tr < TR; ++tr) {
    const int e = e0 + 16 * tr + i;
    wbase[tr] = e < E ? (uint32_t)e * (uint32_t)(d * 4) + (uint32_t)(8 * kg) * 4u : kOOB;
  }
#pragma unroll
  for (int tx = 0; tx < TX; ++tx) {
    const int m = m0 + 16 * tx + i;
    xbase[tx] = m < M ? (uint32_t)m * (uint32_t)(d * EL) + (uint32_t)(8 * kg * EL) : kOOB;
  }
  u32x4 wr[NR][TR][2], xr[NR][TX][EL / 2];
  // iteration it = range q, its r-th slice c = q + 16 r (ranges outermost)
  auto issue = [&](int it, int p) {
    const int q = it / nper, r = it - q * nper, c = q + kRqRanges * r;
    const bool ok = it < total && c < nsl;
    // a dead slice adds kDead to every lane's offset (one uniform value, no
    // per-lane select, which the compiler turns into branches): both
    // operands are under 2^30 bytes (checked by the host), so those loads
    // read zeros
    const uint32_t wstep = ok ? (uint32_t)c * 128u : kDead;
    const uint32_t xstep = ok ? (uint32_t)c * (uint32_t)(32 * EL) : kDead;
#pragma unroll
    for (int tr = 0; tr < TR; ++tr) {
      const uint32_t o = wbase[tr] + wstep;
      wr[p][tr][0] = buf_load16(wres, o);
      wr[p][tr][1] = buf_load16(wres, o + 16);
    }
#pragma unroll
    for (int tx = 0; tx < TX; ++tx) {
      const uint32_t o = xbase[tx] + xstep;
#pragma unroll
      for (int h = 0; h < EL / 2; ++h) xr[p][tx][h] = buf_load16(xres, o + 16 * h);
    }
  };
  f32x4 acc[TR][TX], sum[TR][TX];
#pragma unroll
  for (int tr = 0; tr < TR; ++tr)
#pragma unroll
    for (int tx = 0; tx < TX; ++tx) acc[tr][tx] = sum[tr][tx] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  // the slots are issued in order (the loop's load waits count on it)
  for (int p = 0; p < NR; ++p) {
    issue(p, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it0 = 0; it0 < total; it0 += NR) {
#pragma unroll
    for (int p = 0; p < NR; ++p) {
      const int it = it0 + p;
      bf16x8 a[TR][3];
#pragma unroll
      for (int tr = 0; tr < TR; ++tr) {
        float wv8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) wv8[t] = __uint_as_float(wr[p][tr][t >> 2][t & 3]);
        split3_x8(wv8, a[tr][0], a[tr][1], a[tr][2]);
      }
#pragma unroll
      for (int tx = 0; tx < TX; ++tx) {
        bf16x8 b[NP];
        if constexpr (XBF16) {
          b[0] = bits_to_bf16x8(xr[p][tx][0]);
        } else {
          float xv8[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) xv8[t] = __uint_as_float(xr[p][tx][t >> 2][t & 3]);
          split3_x8(xv8, b[0], b[1], b[2]);
        }
#pragma unroll
        for (int tr = 0; tr < TR; ++tr) acc[tr][tx] = rq_chain<NP>(a[tr], b, acc[tr][tx]);
      }
      issue(it + NR, p);
      __builtin_amdgcn_sched_barrier(0);
      if ((it + 1) % nper == 0) {  // range q = it / nper is complete: add it in range order
        const bool first = it < nper;
#pragma unroll
        for (int tr = 0; tr < TR; ++tr)
#pragma unroll
          for (int tx = 0; tx < TX; ++tx) {
#pragma unroll
            for (int t = 0; t < 4; ++t) sum[tr][tx][t] = first ? acc[tr][tx][t] : sum[tr][tx][t] + acc[tr][tx][t];
            acc[tr][tx] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  }
  // lane (j, g) holds D[4 g + t][j]: router row e0 + 16 tr + 4 g + t, x row m0 + 16 tx + j
#pragma unroll
  for (int tr = 0; tr < TR; ++tr)
#pragma unroll
    for (int tx = 0; tx < TX; ++tx)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = e0 + 16 * tr + 4 * kg + t, m = m0 + 16 * tx + i;
        if (e < E && m < M) logits[(int64_t)m * E + e] = sum[tr][tx][t];
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
  topk_row_any<NPL>(logits + (int64_t)m * E, E, k, lists[wv], lane, id, wt);
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

template <int XBF16, int TR, int TX>
static void launch_logits_tiles(const void *x, const float *w_router, float *logits, int M, int d, int E,
                                hipStream_t stream) {
  hipLaunchKernelGGL((router_mfma_tile_kernel<XBF16, 4, TR, TX>),
                     dim3((E + 16 * TR - 1) / (16 * TR), (M + 16 * TX - 1) / (16 * TX)), dim3(64), 0, stream, x,
                     w_router, M, d, E, logits);
}

template <int XBF16>
static void launch_logits_mfma(const void *x, const float *w_router, float *logits, int M, int d, int E,
                               hipStream_t stream) {
  // router x row tiles per wave by row count, measured at E = 896, d = 7168
  // (1 x 2, 1 x 4, 2 x 2 and 2 x 4 tiles from 200 to 1,533 rows): bf16 x
  // 270 rows 60 us, 512 rows 85 us, 768 rows 112 us, 1,533 rows 166 us;
  // fp32 x 270 rows 107 us, 768 rows 166 us, 1,533 rows 260 us.  The
  // arithmetic of a logit does not depend on the tiles.
  if constexpr (XBF16) {
    if (M <= 288) launch_logits_tiles<XBF16, 1, 2>(x, w_router, logits, M, d, E, stream);
    else if (M <= 512) launch_logits_tiles<XBF16, 1, 4>(x, w_router, logits, M, d, E, stream);
    else launch_logits_tiles<XBF16, 2, 4>(x, w_router, logits, M, d, E, stream);
  } else {
    if (M <= 384) launch_logits_tiles<XBF16, 1, 2>(x, w_router, logits, M, d, E, stream);
    else if (M <= 768) launch_logits_tiles<XBF16, 2, 2>(x, w_router, logits, M, d, E, stream);
    else launch_logits_tiles<XBF16, 2, 4>(x, w_router, logits, M, d, E, stream);
  }
}

template <int XBF16, int RW, int MCH, int KC, int XS>
static void launch_logits_shape(const void *x, const float *w_router, float *logits, int M, int d, int E,
                                hipStream_t stream) {
  hipLaunchKernelGGL((router_logits_kernel<XBF16, RW, MCH, KC, XS>), dim3((E + RW - 1) / RW), dim3(LG_THREADS * XS),
                     0, stream, x, w_router, M, d, E, logits);
}

template <int XBF16>
static void launch_logits(const void *x, const float *w_router, float *logits, int M, int d, int E,
                          hipStream_t stream) {
  // (router rows, x rows per set, chunks per pass, sets) by row count; a
  // sweep of 20 shapes at E = 896, d = 7168, bf16 x (moe_route, logits +
  // top-k, bit-identical logits throughout) kept: 2 and 4 rows 11.7 / 12.2 us
  // (one set: 12.4 / 13.5), 8 rows 13.9 (15.5), 16 rows 17.6 (21.0); two or
  // four sets give each router row more independent waves with shorter row
  // lists.  The arithmetic of a logit never changes.
  if (M == 1) launch_logits_shape<XBF16, 1, 1, 8, 1>(x, w_router, logits, M, d, E, stream);
  else if (M <= 4) launch_logits_shape<XBF16, 2, 2, 4, 2>(x, w_router, logits, M, d, E, stream);
  else if (M <= 8) launch_logits_shape<XBF16, 2, 4, 1, 2>(x, w_router, logits, M, d, E, stream);
  else launch_logits_shape<XBF16, 4, 8, 1, 2>(x, w_router, logits, M, d, E, stream);
}

int logits_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E,
                  hipStream_t stream) {
  if (M > kRqMaxRows) {
    if (x_bf16) launch_logits_mfma<1>(x, w_router, logits, M, d, E, stream);
    else launch_logits_mfma<0>(x, w_router, logits, M, d, E, stream);
  } else {
    if (x_bf16) launch_logits<1>(x, w_router, logits, M, d, E, stream);
    else launch_logits<0>(x, w_router, logits, M, d, E, stream);
  }
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
