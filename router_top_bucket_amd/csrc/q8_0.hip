// Q8_0 spine matmul Y[M x N] = X[M x K] . W^T, W stored as int8 [N x K] and
// one fp16 scale per 32 consecutive K ("A drafter that leaves the answer
// unchanged", "Run Kimi 3.1 locally on one GPU": the spine's matrix multiplies
// load each weight once for up to eight rows).
//
// Every weight is read once per launch for all M (<= 8) rows: the rows are
// the 16 columns of an MFMA B operand (columns >= M are zero).  int8 values are
// exact in bf16; X is split exactly into three bf16 parts (truncation: hi takes
// the top 8 significant bits, mid the next 8 of the remainder, lo the rest), so
// each block's MFMA products are exact.  Per 32-block: P = A.(hi+mid+lo) with a
// fresh accumulator, then acc += P * scale.  Workgroup = 4 waves, each a fixed
// quarter of K's blocks, summed in wave order; nothing depends on M.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int Q8_WAVES = 4;

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, sizeof(v));
  return (float)v;
}

// bf16 bits of an integer in [-128, 127] (exact).
__device__ __forceinline__ uint32_t i8_to_bf16_bits(int v) { return __float_as_uint((float)v) >> 16; }

// split fp32 into three bf16 parts by truncation; v == hi + mid + lo exactly
__device__ __forceinline__ void split3_trunc(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  const uint32_t u = __float_as_uint(v);
  hi = u >> 16;
  const float r1 = v - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t u1 = __float_as_uint(r1);
  mid = u1 >> 16;
  const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
  lo = __float_as_uint(r2) >> 16;
}

template <int RT>
__global__ __launch_bounds__(Q8_WAVES * 64) void q8_0_kernel(const float *__restrict__ X, int M, int K,
                                                             const int8_t *__restrict__ wq,
                                                             const uint16_t *__restrict__ ws, int N,
                                                             float *__restrict__ Y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int nbk = K >> 5;                 // blocks per row
  const int srow = nbk + 2;               // padded fp16 row of scales (halves)
  uint16_t *sc_lds = (uint16_t *)smem;    // [RT*16][srow]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * RT * 16;
  const int rows_here = (N - n0) < RT * 16 ? (N - n0) : RT * 16;

  for (int idx = tid; idx < RT * 16 * nbk; idx += Q8_WAVES * 64) {
    const int rr = idx / nbk, cc = idx % nbk;
    sc_lds[rr * srow + cc] = rr < rows_here ? ws[(int64_t)(n0 + rr) * nbk + cc] : (uint16_t)0;
  }

  const bool col_ok = r < M;
  const float *xrow = X + (int64_t)(col_ok ? r : 0) * K;
  const int8_t *arow[RT];
  bool aok[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = n0 + 16 * t + r;
    aok[t] = row < N;
    arow[t] = wq + (int64_t)(aok[t] ? row : 0) * K;
  }
  const int b_begin = (wv * nbk) / Q8_WAVES, b_end = ((wv + 1) * nbk) / Q8_WAVES;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  constexpr int PF = 4;  // blocks of weights in flight per lane
  u32x2 a_buf[PF][RT];
#pragma unroll
  for (int p = 0; p < PF; ++p)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int b = b_begin + p;
      a_buf[p][t] = (aok[t] && b < b_end) ? *(const u32x2 *)(arow[t] + 32 * b + 8 * q) : u32x2{0u, 0u};
    }

  for (int b0 = b_begin; b0 < b_end; b0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int b = b0 + p;
      if (b >= b_end) break;
      u32x2 a_cur[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        a_cur[t] = a_buf[p][t];
        const int bn = b + PF;
        a_buf[p][t] = (aok[t] && bn < b_end) ? *(const u32x2 *)(arow[t] + 32 * bn + 8 * q) : u32x2{0u, 0u};
      }
      // B: X[col r][32b + 8q .. +8] split in three exact bf16 parts
      f32x4 x0 = f32x4{0.f, 0.f, 0.f, 0.f}, x1 = x0;
      if (col_ok) {
        x0 = *(const f32x4 *)(xrow + 32 * b + 8 * q);
        x1 = *(const f32x4 *)(xrow + 32 * b + 8 * q + 4);
      }
      uint32_t hi[8], mi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        split3_trunc(x0[e], hi[e], mi[e], lo[e]);
        split3_trunc(x1[e], hi[e + 4], mi[e + 4], lo[e + 4]);
      }
      u32x4 ph, pm, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
        pm[e] = mi[2 * e] | (mi[2 * e + 1] << 16);
        pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
      }
      const bf16x8 bh = bits_to_bf16x8(ph), bm = bits_to_bf16x8(pm), bl = bits_to_bf16x8(pl);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        u32x4 av;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t wdw = a_cur[t][h];
          const uint32_t e0 = i8_to_bf16_bits((int)(int8_t)(wdw & 0xFF));
          const uint32_t e1 = i8_to_bf16_bits((int)(int8_t)((wdw >> 8) & 0xFF));
          const uint32_t e2 = i8_to_bf16_bits((int)(int8_t)((wdw >> 16) & 0xFF));
          const uint32_t e3 = i8_to_bf16_bits((int)(int8_t)(wdw >> 24));
          av[2 * h] = e0 | (e1 << 16);
          av[2 * h + 1] = e2 | (e3 << 16);
        }
        const bf16x8 a = bits_to_bf16x8(av);
        f32x4 p = mfma16x16x32(a, bh, f32x4{0.f, 0.f, 0.f, 0.f});
        p = mfma16x16x32(a, bm, p);
        p = mfma16x16x32(a, bl, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * t + 4 * q + i;
          const float s = half_bits_to_f32(sc_lds[rr * srow + b]);
          acc[t][i] = __builtin_fmaf(p[i], s, acc[t][i]);
        }
      }
    }
  }

  // fixed-order sum of the 4 K quarters
  __syncthreads();
  float *red = (float *)smem;  // [wave][RT*4][64]
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wv * RT * 4 + t * 4 + i) * 64 + lane] = acc[t][i];
  __syncthreads();
  for (int idx = tid; idx < RT * 4 * 64; idx += Q8_WAVES * 64) {
    const int ln = idx & 63, ti = idx >> 6;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < Q8_WAVES; ++w) v += red[(w * RT * 4 + ti) * 64 + ln];
    const int col = ln & 15;
    const int t = ti >> 2, i = ti & 3;
    const int row = n0 + 16 * t + 4 * (ln >> 4) + i;
    if (col < M && row < N) Y[(int64_t)col * N + row] = v;
  }
}

template <int RT>
static int q8_launch_rt(const float *X, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *Y,
                        hipStream_t stream) {
  const int nbk = K / 32;
  const size_t sc = (size_t)RT * 16 * (nbk + 2) * sizeof(uint16_t);
  const size_t rd = (size_t)Q8_WAVES * RT * 4 * 64 * sizeof(float);
  const size_t smem = sc > rd ? sc : rd;
  const int grid = (N + RT * 16 - 1) / (RT * 16);
  hipLaunchKernelGGL(q8_0_kernel<RT>, dim3(grid), dim3(Q8_WAVES * 64), smem, stream, X, M, K, wq, ws, N, Y);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int q8_0_launch(const float *X, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *Y,
                hipStream_t stream) {
  if (N <= 16384) return q8_launch_rt<2>(X, M, K, wq, ws, N, Y, stream);
  return q8_launch_rt<4>(X, M, K, wq, ws, N, Y, stream);
}

}  // namespace moe
