// Q8_0 spine matmul Y[M x N] = X[M x K] . W^T, W stored as int8 [N x K] and
// one fp16 scale per 32 consecutive K.  Up to 8 rows of X share one pass
// over W, so each weight byte leaves HBM once per call, not once per row
// ("Run Kimi 3.1 locally on one GPU", sections "A drafter that leaves the
// answer unchanged" and "One GPU, three storage tiers").
//
// Arithmetic (fixed for a given K and N, independent of M and of the launch
// shape below): for output row n and X row m, each 32-block b contributes
//   P_p = sum_{c in b} q[n,c] * x_p[m,c]        (one MFMA column, fresh C = 0)
// for the two bf16 parts of x (q8_split2: x_0 = x to the nearest bf16, x_1 =
// the remainder to the nearest bf16, |x - x_0 - x_1| <= 2^-18 |x|; int8 is
// exact in bf16, so every product is exact on those parts), and
//   A_p <- fma(P_p, s[n,b], A_p)                 (v_fma_mix: fp16 scale, one rounding)
// runs over the blocks of a K part in ascending order.  The KS K parts are
// summed in part order per p, and y = A_0 + A_1.
//
// Mapping.  A wave owns RT tiles of 16 weight rows and one K part; a step is
// 64 K (two blocks).  Lane (r, q) loads 16 bytes of row r at K offset
// 64s + 16q, so lanes q < 2 hold block 2s and q >= 2 block 2s+1; one
// v_permlane32_swap per dword pair regroups them so each block's 32 values
// sit 8 per lane group in the order {0, 16, 8, 24} + 0..7, the MFMA A layout.
// The MFMA B operand has one column per (m, p): column 2m + p, so M <= 8 needs
// one 16-column MFMA per block.  The wave splits X for the step
// once (EPL elements per lane) into its own LDS area in that layout, and every
// tile of the wave reads it back.  Scales: once per 16 steps lane (r, q)
// loads the 8 fp16 scales of row r for blocks 2 s0 + 8q .. +7 of the chunk
// (so each 64-byte piece of a scale row is fetched by one instruction); a
// bpermute hands each lane the dword of output row 4q' + i for the step.
// Every global load is an unconditional buffer load (dead steps and masked
// lanes read past the resource and get zeros).
//
// Weight order: rows (row n's K bytes contiguous) or tiles (N % 16 == 0:
// block b of row n at ((n/16)*(K/32) + b)*512 + (n%16)*32, so the 16 rows of
// a tile keep each block's 32-byte pieces side by side and one step of a
// wave, 16 rows x 64 bytes, is one contiguous kilobyte).  Every lane loads the
// same bytes in both orders, so the results are bit-identical.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int Q8_MAX_WAVES = 8;
constexpr int kQ8Chunk = 16;  // steps per scale load (32 blocks)

// Upper halves of two fp32 bit patterns as one packed pair (a low, b high).
__device__ __forceinline__ uint32_t q8_pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Four int8 (element 0 in byte 0) as four bf16, exact.
__device__ __forceinline__ u32x2 q8_i8x4_to_bf16(uint32_t w) {
  const float f0 = (float)(int8_t)w, f1 = (float)(int8_t)(w >> 8);
  const float f2 = (float)(int8_t)(w >> 16), f3 = (float)(int8_t)(w >> 24);
  return u32x2{q8_pack_hi16(__float_as_uint(f0), __float_as_uint(f1)),
               q8_pack_hi16(__float_as_uint(f2), __float_as_uint(f3))};
}

// Round-to-nearest-even of an fp32 pattern to bf16, returned as the fp32
// pattern of that bf16 value (upper 16 bits; finite inputs).
__device__ __forceinline__ uint32_t q8_round_bf16(uint32_t u) {
  return ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) << 16;
}

// v ~= hi + lo: hi is v to the nearest bf16 and lo the remainder (an exact
// fp32 difference) to the nearest bf16, so |v - hi - lo| <= 2^-18 |v|; each
// part is the upper 16 bits of the returned fp32 pattern.
__device__ __forceinline__ void q8_split2(float v, uint32_t &hi, uint32_t &lo) {
  hi = q8_round_bf16(__float_as_uint(v));
  lo = q8_round_bf16(__float_as_uint(v - __uint_as_float(hi)));
}

// The same split for two values at once with the paired round-to-nearest-even
// convert (v_cvt_pk_bf16_f32): hi and lo each hold the two parts packed
// (x0's in the low half), bit for bit the parts q8_split2 gives.
typedef float q8_f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
__device__ __forceinline__ uint32_t q8_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((q8_f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ void q8_split2_pk(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = q8_pk_bf16(x0, x1);
  lo = q8_pk_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ float q8_f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float q8_f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// LDS of one wave: the X fragments of one step (2 blocks x 4 lane groups x
// 16*NMF columns x 16 B, then a 16-byte dummy slot for masked writes); after
// the main loop the same bytes hold the wave's partial sums [RT][NMF][4][65].
// Column c of fragment row b = 4 jb + g sits in 16-byte slot c ^ q8_swz(b)
// of its 16-column group: the X split writes one column of all eight rows
// per eight lanes, and rows 256 bytes apart would put those writes on the
// same banks; a fragment read (16 consecutive columns of one row) stays a
// permutation of 16 slots.
__device__ __forceinline__ constexpr int q8_swz(int b) { return (b & 1) | ((b >> 1) << 2); }
template <int RT, int NMF>
struct Q8Lds {
  static constexpr int kCols = 16 * NMF;
  static constexpr int kFrag = 2 * 4 * kCols * 16;
  static constexpr int kPart = RT * NMF * 4 * 65 * 4;
  static constexpr int kWave = ((kFrag + 16 > kPart ? kFrag + 16 : kPart) + 15) / 16 * 16;
};

template <int RT, int PF, int EPL, int NMF, bool MASKED, int WPE>
__global__ __launch_bounds__(Q8_MAX_WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void q8_0_kernel(const float *__restrict__ X, int M, int K,
                                                                 const int8_t *__restrict__ wq,
                                                                 const uint16_t *__restrict__ ws, int N,
                                                                 float *__restrict__ Y, int KS, int RG, int tiled) {
  static_assert(kQ8Chunk % PF == 0, "ring depth divides the scale chunk");
  static_assert(EPL == 1 || EPL == 2 || EPL == 4 || EPL == 8, "X elements per lane");
  using L = Q8Lds<RT, NMF>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int rg = wv / KS, part = wv - rg * KS;
  uint8_t *wl = smem + wv * L::kWave;
  const int nb = K >> 5, ns = (nb + 1) >> 1;
  const int row0 = (blockIdx.x * RG + rg) * RT * 16;

  f32x4 acc[RT][NMF];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) acc[t][mf] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (row0 < N) {  // uniform per wave
    const int s_begin = (int)((int64_t)part * ns / KS), s_end = (int)((int64_t)(part + 1) * ns / KS);
    const int b_end = 2 * s_end < nb ? 2 * s_end : nb;
    const int nchunks = (s_end - s_begin + kQ8Chunk - 1) / kQ8Chunk;
    const int rows_here = N - row0 < RT * 16 ? N - row0 : RT * 16;

    // weights and scales of this wave's rows; rows past N read row N-1
    const rsrc_t wrs = make_rsrc(wq + (int64_t)row0 * K, (uint32_t)rows_here * (uint32_t)K);
    const rsrc_t srs = make_rsrc(ws + (int64_t)row0 * nb, (uint32_t)rows_here * (uint32_t)nb * 2u);
    uint32_t woff[RT], soff[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rr = 16 * t + r < rows_here ? 16 * t + r : rows_here - 1;
      woff[t] = tiled ? ((uint32_t)(rr >> 4) * (uint32_t)nb + (uint32_t)(q >> 1)) * 512u + (uint32_t)(rr & 15) * 32u +
                            16u * (uint32_t)(q & 1)
                      : (uint32_t)rr * (uint32_t)K + 16u * q;
      soff[t] = (uint32_t)rr * (uint32_t)nb * 2u;
    }
    // X: lane handles row xm, elements xk .. xk+EPL-1 of each step's 64
    constexpr int LPR = 64 / EPL;
    const int xm = lane / LPR, xk = (lane % LPR) * EPL;
    const rsrc_t xrs = make_rsrc(X, (uint32_t)M * (uint32_t)K * 4u);
    const uint32_t xoff = xm < M ? ((uint32_t)xm * (uint32_t)K + (uint32_t)xk) * 4u : kOOB;
    // where this lane's split goes: block j, lane group g, column 3 xm + p
    const int xj = xk >> 5, xg8 = (xk & 31) >> 3, xe = xk & 7;
    const int xg = ((xg8 & 1) << 1) | (xg8 >> 1);
    // (x_0 in column 2 xm, x_1 in column 2 xm + 1; both < 16)
    const int xb = xj * 4 + xg;
    const uint32_t xdst = xm < M ? (uint32_t)((xb * L::kCols + ((2 * xm) ^ q8_swz(xb))) * 16 + 2 * xe) : (uint32_t)L::kFrag;
    const uint32_t xdst_lo =
        xm < M ? (uint32_t)((xb * L::kCols + ((2 * xm + 1) ^ q8_swz(xb))) * 16 + 2 * xe) : (uint32_t)L::kFrag;
    // fragment reads: lane (r, q) reads column 16 mf + r of row 4 jb + q
    uint32_t frd[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) frd[jb] = (uint32_t)(((4 * jb + q) * L::kCols + (r ^ q8_swz(4 * jb + q))) * 16);
    // scale bpermute source addresses: output row 4q + i lives in lane 4q + i
    int baddr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) baddr[i] = (4 * q + i) * 4;

    // zero the fragment area once: columns >= 3M are never written
#pragma unroll
    for (int i = 0; i < L::kFrag / (64 * 16); ++i)
      *(u32x4 *)(wl + (i * 64 + lane) * 16) = u32x4{0u, 0u, 0u, 0u};

    u32x4 wr[PF][RT];
    uint32_t xr[PF][EPL];
    uint32_t sc_cur[RT][4], sc_nxt[RT][4];

    const uint32_t wsz = tiled ? 1024u : 64u;  // weight bytes a step advances by
    auto issue = [&](int s, int slot) {
      const bool live_step = s < s_end;  // uniform
      const uint32_t wstep = live_step ? wsz * (uint32_t)s : kDead;
      const uint32_t xstep = live_step ? 256u * (uint32_t)s : kDead;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        uint32_t o = woff[t];
        if constexpr (MASKED) o = 2 * s + (q >> 1) < b_end ? o : kOOB;
        wr[slot][t] = buf_load16_stream(wrs, o + wstep);
      }
      uint32_t xo = xoff;
      if constexpr (MASKED) xo = 2 * s + xj < b_end ? xo : kOOB;
      xo += xstep;
      if constexpr (EPL == 8) {
        const u32x4 a = buf_load16(xrs, xo), b = buf_load16(xrs, xo + 16u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xr[slot][e] = a[e];
          xr[slot][4 + e] = b[e];
        }
      } else if constexpr (EPL == 4) {
        const u32x4 a = buf_load16(xrs, xo);
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[slot][e] = a[e];
      } else if constexpr (EPL == 2) {
        const u32x2 a = buf_load8(xrs, xo);
        xr[slot][0] = a[0];
        xr[slot][1] = a[1];
      } else {
        xr[slot][0] = buf_load4(xrs, xo);
      }
    };
    // scales of chunk c: lane (r, q) takes the 8 fp16 of row r for blocks
    // 2 s_begin + 32 c + 8 q .. +7 (one 64-byte piece of the row per 4 lanes)
    auto load_scales = [&](int c, uint32_t (&sc)[RT][4]) {
      const int b = 2 * s_begin + 2 * kQ8Chunk * c + 8 * q;
      const uint32_t gs = c < nchunks ? 0u : kDead;  // uniform
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if constexpr (!MASKED) {
          const u32x4 v = buf_load16(srs, soff[t] + 2u * (uint32_t)b + gs);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[t][e] = v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int b0 = b + 2 * e;
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                srs, (b0 < b_end ? soff[t] + 2u * (uint32_t)b0 : kOOB) + gs, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                srs, (b0 + 1 < b_end ? soff[t] + 2u * (uint32_t)b0 + 2u : kOOB) + gs, 0, 0);
            sc[t][e] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
        }
      }
    };

    load_scales(0, sc_cur);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      issue(s_begin + i, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // start the loop with nothing in flight, so the waits inside it are the
    // steady-state ones (one slot's loads at a time); the empty asm keeps the
    // compiler from sinking the prefill loads below the wait
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    asm volatile("" ::: "memory");

    // a do-while: every part has at least one step (at most ns parts), and a
    // loop guard would let the compiler sink the prefill into the guarded block
    int c = 0;
    do {
      load_scales(c + 1, sc_nxt);
#pragma unroll
      for (int u = 0; u < kQ8Chunk; ++u) {
        const int s = s_begin + kQ8Chunk * c + u;
        const int slot = u % PF;
        // 1. split this step's X into the fragment area
        {
          if constexpr (EPL == 1) {
            uint32_t hp, lp;
            q8_split2(__uint_as_float(xr[slot][0]), hp, lp);
            *(uint16_t *)(wl + xdst) = (uint16_t)(hp >> 16);
            *(uint16_t *)(wl + xdst_lo) = (uint16_t)(lp >> 16);
          } else {
            constexpr int NP = EPL / 2;  // packed pairs
            uint32_t hp[NP], lp[NP];
#pragma unroll
            for (int e = 0; e < NP; ++e)
              q8_split2_pk(__uint_as_float(xr[slot][2 * e]), __uint_as_float(xr[slot][2 * e + 1]), hp[e], lp[e]);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const uint32_t *src = p == 0 ? hp : lp;
              const uint32_t d = p == 0 ? xdst : xdst_lo;
              if constexpr (EPL == 8)
                *(u32x4 *)(wl + d) = u32x4{src[0], src[1], src[2], src[3]};
              else if constexpr (EPL == 4)
                *(u32x2 *)(wl + d) = u32x2{src[0], src[1]};
              else
                *(uint32_t *)(wl + d) = src[0];
            }
          }
        }
        // 2. weights of both blocks as bf16 A fragments
        bf16x8 a[RT][2];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const u32x4 v = wr[slot][t];
          const auto s02 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
          const auto s13 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
          const u32x2 a0 = q8_i8x4_to_bf16(s02[0]), a1 = q8_i8x4_to_bf16(s13[0]);
          const u32x2 b0 = q8_i8x4_to_bf16(s02[1]), b1 = q8_i8x4_to_bf16(s13[1]);
          a[t][0] = bits_to_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]});
          a[t][1] = bits_to_bf16x8(u32x4{b0[0], b0[1], b1[0], b1[1]});
        }
        // 3. this step's scales (row 4q + i; low half block 2s, high half 2s+1)
        uint32_t sv[RT][4];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sv[t][i] = (uint32_t)__builtin_amdgcn_ds_bpermute(baddr[i] + 64 * (u >> 2), (int)sc_cur[t][u & 3]);
        // 4. per block: fresh product, scaled into the accumulators
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          bf16x8 bfr[NMF];
#pragma unroll
          for (int mf = 0; mf < NMF; ++mf)
            bfr[mf] = bits_to_bf16x8(*(const u32x4 *)(wl + frd[jb] + (uint32_t)(16 * mf * 16)));
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int mf = 0; mf < NMF; ++mf) {
              const f32x4 p = mfma16x16x32(a[t][jb], bfr[mf], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float sc = jb == 0 ? q8_f16_lo(sv[t][i]) : q8_f16_hi(sv[t][i]);
                acc[t][mf][i] = __builtin_fmaf(p[i], sc, acc[t][mf][i]);
              }
            }
        }
        // 5. refill the slot
        issue(s + PF, slot);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc_cur[t][e] = sc_nxt[t][e];
    } while (++c < nchunks);
  }

  // partial sums of this wave -> LDS (its own area), then a fixed-order sum
  float *pw = (float *)wl;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[((t * NMF + mf) * 4 + i) * 65 + lane] = acc[t][mf][i];
  lds_barrier();
  const int per_rg = RT * 16 * M;
  for (int it = tid; it < RG * per_rg; it += blockDim.x) {
    const int g = it / per_rg, rem = it - g * per_rg;
    const int m = rem / (RT * 16), row = rem - m * (RT * 16);
    const int n = (blockIdx.x * RG + g) * RT * 16 + row;
    if (n >= N) continue;
    const int t = row >> 4, qq = (row >> 2) & 3, i = row & 3;
    float part_sum[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int col = 2 * m + p, mf = col >> 4, c = col & 15;
      const int idx = ((t * NMF + mf) * 4 + i) * 65 + 16 * qq + c;
      float v = ((const float *)(smem + (g * KS) * L::kWave))[idx];
      for (int w = 1; w < KS; ++w) v += ((const float *)(smem + (g * KS + w) * L::kWave))[idx];
      part_sum[p] = v;
    }
    Y[(int64_t)m * N + n] = part_sum[0] + part_sum[1];
  }
}

// Launch one configuration.  KS K parts x RG row groups = waves per workgroup;
// WPE is the register budget as a target of resident waves per SIMD.
template <int RT, int PF, int EPL, int NMF, bool MASKED, int WPE>
static int q8_run(const float *X, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *Y, int KS,
                  int RG, int tiled, hipStream_t stream) {
  using L = Q8Lds<RT, NMF>;
  if (KS < 1 || RG < 1 || KS * RG > Q8_MAX_WAVES || M > EPL || 2 * M > 16 * NMF) return -3;
  const size_t smem = (size_t)KS * RG * L::kWave;
  auto kern = q8_0_kernel<RT, PF, EPL, NMF, MASKED, WPE>;
  if (smem > 65536 &&
      hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return -3;
  const int64_t groups = ((int64_t)N + RT * 16 - 1) / (RT * 16);
  const int64_t grid = (groups + RG - 1) / RG;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KS * RG), smem, stream, X, M, K, wq, ws, N, Y, KS, RG,
                     tiled);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// K parts depend on K and N only, so every M sees the same reduction order.
// The fast path needs whole 16-step chunks per part.
static int q8_k_parts(int K, int N) {
  const int ns = (K / 32 + 1) / 2;
  const int64_t tiles = ((int64_t)N + 15) / 16;
  const int target = tiles >= 4096 ? 1 : Q8_MAX_WAVES;
  if (ns % kQ8Chunk == 0) {
    for (int ks = target; ks >= 1; --ks)
      if ((ns / kQ8Chunk) % ks == 0) return ks;
  }
  return target < ns ? target : ns;
}

static bool q8_fast_path(int K, int KS, const uint16_t *ws) {
  const int nb = K / 32, ns = (nb + 1) / 2;
  return nb % 8 == 0 && ns % (kQ8Chunk * KS) == 0 && reinterpret_cast<uintptr_t>(ws) % 16 == 0;
}

// Launch shapes by X rows and weight size (measured on MI355X); none of them
// changes the arithmetic, which depends on K and N only.
int q8_0_launch(const float *X, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *Y, int tiled,
                hipStream_t stream) {
  const int KS = q8_k_parts(K, N);
  const int RG = Q8_MAX_WAVES / KS >= 4 ? 4 : 1;
  const bool big = ((int64_t)N + 15) / 16 >= 4096;
  if (!q8_fast_path(K, KS, ws)) {
    if (M <= 1) return q8_run<2, 4, 1, 1, true, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
    if (M <= 2) return q8_run<2, 4, 2, 1, true, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
    if (M <= 4) return q8_run<2, 4, 4, 1, true, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
    if (M <= 5) return q8_run<2, 4, 8, 1, true, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
    return q8_run<2, 4, 8, 1, true, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
  }
  if (M <= 1)
    return big ? q8_run<2, 4, 1, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream)
               : q8_run<1, 4, 1, 1, false, 6>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
  if (M <= 2)
    return big ? q8_run<2, 4, 2, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream)
               : q8_run<1, 4, 2, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
  if (M <= 4)
    return big ? q8_run<2, 4, 4, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream)
               : q8_run<2, 2, 4, 1, false, 5>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
  if (M <= 5)
    return big ? q8_run<2, 4, 8, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream)
               : q8_run<2, 2, 8, 1, false, 4>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
  return big ? q8_run<4, 2, 8, 1, false, 1>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream)
             : q8_run<2, 2, 8, 1, false, 4>(X, M, K, wq, ws, N, Y, KS, RG, tiled, stream);
}

}  // namespace moe
