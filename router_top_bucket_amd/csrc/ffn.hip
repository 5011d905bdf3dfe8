// Expert FFN over bucketed slots: y = W_down (silu(W_gate x) * (W_up x)) with
// MXFP4 weights, each expert's weights streamed once for all rows of its
// bucket ("A drafter that leaves the answer unchanged", "Run Kimi 3.1 locally
// on one GPU": a block reads each expert once for all its rows).
//
// Work unit: a "group" = one expert and up to 16 of its slots (a bucket
// segment of <= 16 positions of perm).  With M <= 16 rows every active expert
// is exactly one group; for more rows a plan kernel cuts each segment into
// pieces of 16.  Each group is one 16-column MFMA operand: column n holds the
// n-th slot of the group, so a slot's arithmetic never depends on which other
// slots share its group (an MFMA output column depends only on its own input
// column) or on how many there are.
//
// Arithmetic: weights are decoded exactly to bf16 (E2M1 x 2^k) with gfx950's
// scaled FP4 convert; x in bf16 is used as is, fp32 x and the fp32 hidden h
// are split exactly into three bf16 parts (hi + mid + lo), so every MFMA
// product is exact and only fp32 accumulation rounds.  The K order of every
// accumulation is fixed by d and f alone.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kGroupCols = 16;

// ------------------------------------------------------------------ groups
struct GroupSrc {
  const int32_t *offsets;  // direct mode: bucket offsets
  const int32_t *active;   // direct mode
  const int32_t *n_active; // direct mode
  const int4 *groups;      // plan mode: {expert, start, count, 0}
  const int32_t *n_groups; // plan mode
};

__device__ __forceinline__ bool load_group(const GroupSrc &src, int g, int &expert, int &start, int &count) {
  if (src.groups) {
    if (g >= *src.n_groups) return false;
    int4 v = src.groups[g];
    expert = v.x; start = v.y; count = v.z;
  } else {
    if (g >= *src.n_active) return false;
    expert = src.active[g];
    start = src.offsets[expert];
    count = src.offsets[expert + 1] - start;
  }
  count = count < kGroupCols ? count : kGroupCols;
  return count > 0;
}

// One workgroup: cut every active expert's segment into groups of <= 16 slots.
__global__ __launch_bounds__(1024) void plan_groups_kernel(const int32_t *offsets, const int32_t *active,
                                                           const int32_t *n_active, int4 *groups,
                                                           int32_t *n_groups) {
  __shared__ int32_t wave_tot[16];
  const int na = *n_active;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int running = 0;  // groups emitted by earlier passes
  for (int base = 0; base < na; base += 1024) {
    const int i = base + tid;
    int cnt = 0, ng = 0, e = 0;
    if (i < na) {
      e = active[i];
      cnt = offsets[e + 1] - offsets[e];
      ng = (cnt + kGroupCols - 1) / kGroupCols;
    }
    // inclusive scan of ng over the workgroup
    int v = ng;
    for (int o = 1; o < 64; o <<= 1) {
      int t = __shfl_up(v, o, 64);
      if (lane >= o) v += t;
    }
    if (lane == 63) wave_tot[wv] = v;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
      int t = wave_tot[w];
      if (w < wv) before += t;
      total += t;
    }
    const int excl = running + before + v - ng;
    for (int j = 0; j < ng; ++j) {
      int rem = cnt - j * kGroupCols;
      groups[excl + j] = make_int4(e, offsets[e] + j * kGroupCols, rem < kGroupCols ? rem : kGroupCols, 0);
    }
    running += total;
    __syncthreads();
  }
  if (tid == 0) *n_groups = running;
}

// ------------------------------------------------------------------ gate/up
// Workgroup = (group, tile of 64 rows of f).  8 waves split the d reduction
// into 8 fixed slices of 128-element steps; each wave keeps 4 gate and 4 up
// 16-row accumulator tiles.  Lane l = (r = l%16, q = l/16): for every step
// the lane loads 16 bytes of codes = one 32-element MXFP4 block (row r, block
// q of the step) per tile, and the 64 bytes of x of the same K range for
// column r.  MFMA j (0..3) of a step consumes elements 8j..8j+7 of each
// lane's block.
constexpr int GU_ROWS = 64;
constexpr int GU_WAVES = 8;
constexpr int GU_T = 4;  // 16-row tiles per matrix per wave

template <int XBF16>
__global__ __launch_bounds__(GU_WAVES * 64) void ffn_gateup_kernel(
    const void *__restrict__ x, int d, int f, int kps, int n_slots, const uint8_t *__restrict__ experts,
    int64_t stride, GroupSrc src, const int32_t *__restrict__ perm, int n_ftiles, uint16_t *__restrict__ h_ws) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int g = blockIdx.x / n_ftiles;
  const int ft = blockIdx.x % n_ftiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int i0 = ft * GU_ROWS;
  const int nb = d >> 5;  // scale blocks per row
  const int srow = (nb & 3) ? nb : nb + 4;
  const int64_t plane_c = (int64_t)f * d / 2, plane_s = (int64_t)f * d / 32;
  const uint8_t *rec = experts + (int64_t)expert * stride;
  const uint8_t *gc = rec, *gs = rec + plane_c, *uc = rec + plane_c + plane_s, *us = uc + plane_c;

  // ---- stage the tile's scales (64 gate rows then 64 up rows) in LDS
  const int rows_here = (f - i0) < GU_ROWS ? (f - i0) : GU_ROWS;
  if ((nb & 3) == 0) {
    const int dw_per_row = nb >> 2;
    for (int idx = tid; idx < 2 * GU_ROWS * dw_per_row; idx += GU_WAVES * 64) {
      const int mat = idx / (GU_ROWS * dw_per_row), rem = idx % (GU_ROWS * dw_per_row);
      const int rr = rem / dw_per_row, cc = rem % dw_per_row;
      uint32_t v = 0;
      if (rr < rows_here) v = *(const uint32_t *)((mat ? us : gs) + (int64_t)(i0 + rr) * nb + cc * 4);
      *(uint32_t *)(smem + (mat * GU_ROWS + rr) * srow + cc * 4) = v;
    }
  } else {
    for (int idx = tid; idx < 2 * GU_ROWS * nb; idx += GU_WAVES * 64) {
      const int mat = idx / (GU_ROWS * nb), rem = idx % (GU_ROWS * nb);
      const int rr = rem / nb, cc = rem % nb;
      smem[(mat * GU_ROWS + rr) * srow + cc] = rr < rows_here ? (mat ? us : gs)[(int64_t)(i0 + rr) * nb + cc] : 0;
    }
  }

  // ---- this lane's B column: slot start+r of the group
  const bool col_ok = r < count;
  int64_t xrow = 0;
  if (col_ok) {
    const int t = perm[start + r];
    xrow = (t >= 0 && t < n_slots) ? (int64_t)(t / kps) : 0;
  }

  // ---- A row pointers (tile t: t<4 gate, t>=4 up)
  const uint8_t *arow[2 * GU_T];
  bool aok[2 * GU_T];
#pragma unroll
  for (int t = 0; t < 2 * GU_T; ++t) {
    const int row = i0 + 16 * (t % GU_T) + r;
    aok[t] = row < f;
    arow[t] = (t < GU_T ? gc : uc) + (int64_t)(aok[t] ? row : 0) * (d / 2);
  }

  const int nsteps = (d + 127) >> 7;
  const int s_begin = (wv * nsteps) / GU_WAVES, s_end = ((wv + 1) * nsteps) / GU_WAVES;

  f32x4 acc[2 * GU_T];
#pragma unroll
  for (int t = 0; t < 2 * GU_T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();

  u32x4 a_nxt[2 * GU_T];
  auto load_a = [&](int s, u32x4 *dst) {
    const int kq = (s << 7) + (q << 5);
    const bool kok = kq < d;
#pragma unroll
    for (int t = 0; t < 2 * GU_T; ++t)
      dst[t] = (aok[t] && kok) ? *(const u32x4 *)(arow[t] + (kq >> 1)) : u32x4{0u, 0u, 0u, 0u};
  };
  if (s_begin < s_end) load_a(s_begin, a_nxt);

  for (int s = s_begin; s < s_end; ++s) {
    u32x4 a_cur[2 * GU_T];
#pragma unroll
    for (int t = 0; t < 2 * GU_T; ++t) a_cur[t] = a_nxt[t];
    if (s + 1 < s_end) load_a(s + 1, a_nxt);

    const int kq = (s << 7) + (q << 5);
    const bool kok = kq < d;
    // B operand: x[xrow][kq .. kq+32) as bf16 (3 exact parts for fp32 x)
    bf16x8 b[XBF16 ? 4 : 12];
    if (XBF16) {
      const uint16_t *xp = (const uint16_t *)x + xrow * d + kq;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = (col_ok && kok) ? bits_to_bf16x8(*(const u32x4 *)(xp + 8 * j)) : bits_to_bf16x8(u32x4{0u, 0u, 0u, 0u});
    } else {
      const float *xp = (const float *)x + xrow * d + kq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (col_ok && kok) {
          v0 = *(const f32x4 *)(xp + 8 * j);
          v1 = *(const f32x4 *)(xp + 8 * j + 4);
        }
        uint32_t hi[8], mi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split3_bf16(v0[e], hi[e], mi[e], lo[e]);
          split3_bf16(v1[e], hi[e + 4], mi[e + 4], lo[e + 4]);
        }
        u32x4 ph, pm, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
          pm[e] = mi[2 * e] | (mi[2 * e + 1] << 16);
          pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
        }
        b[3 * j] = bits_to_bf16x8(ph);
        b[3 * j + 1] = bits_to_bf16x8(pm);
        b[3 * j + 2] = bits_to_bf16x8(pl);
      }
    }
    float sc[2 * GU_T];
#pragma unroll
    for (int t = 0; t < 2 * GU_T; ++t)
      sc[t] = e8m0_to_f32(smem[((t / GU_T) * GU_ROWS + 16 * (t % GU_T) + r) * srow + (kok ? (kq >> 5) : 0)]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < 2 * GU_T; ++t) {
        const bf16x8 a = fp4x8_to_bf16(a_cur[t][j], sc[t]);
        if (XBF16) {
          acc[t] = mfma16x16x32(a, b[j], acc[t]);
        } else {
          acc[t] = mfma16x16x32(a, b[3 * j], acc[t]);
          acc[t] = mfma16x16x32(a, b[3 * j + 1], acc[t]);
          acc[t] = mfma16x16x32(a, b[3 * j + 2], acc[t]);
        }
      }
    }
  }

  // ---- fixed-order reduction of the 8 K slices, SwiGLU, exact 3-way split
  __syncthreads();  // scales no longer needed; reuse LDS
  float *red = (float *)smem;  // [wave][32 values][64 lanes]
#pragma unroll
  for (int t = 0; t < 2 * GU_T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wv * 32 + t * 4 + i) * 64 + lane] = acc[t][i];
  __syncthreads();
  for (int idx = tid; idx < GU_T * 4 * 64; idx += GU_WAVES * 64) {
    const int ln = idx & 63, ti = idx >> 6;  // ti = t*4 + i over the gate tiles
    const int t = ti >> 2, i = ti & 3;
    float gsum = 0.f, usum = 0.f;
#pragma unroll
    for (int w = 0; w < GU_WAVES; ++w) {
      gsum += red[(w * 32 + ti) * 64 + ln];
      usum += red[(w * 32 + (t + GU_T) * 4 + i) * 64 + ln];
    }
    const int n = ln & 15;
    const int frow = i0 + 16 * t + 4 * (ln >> 4) + i;
    if (n < count && frow < f) {
      const float h = (gsum / (1.0f + expf(-gsum))) * usum;
      uint32_t hi, mi, lo;
      split3_bf16(h, hi, mi, lo);
      uint16_t *hp = h_ws + (int64_t)(start + n) * 3 * f + frow;
      hp[0] = (uint16_t)hi;
      hp[f] = (uint16_t)mi;
      hp[2 * f] = (uint16_t)lo;
    }
  }
}

// ------------------------------------------------------------------ down
// Workgroup = (group, DN_WAVES * 128 rows of d); each wave owns 8 row tiles of
// 16 and the full f reduction (no split), B = the group's h in three bf16
// planes.  y_slots rows are written directly (each slot by exactly one lane).
constexpr int DN_WAVES = 4;
constexpr int DN_T = 8;
constexpr int DN_ROWS = DN_WAVES * DN_T * 16;

__global__ __launch_bounds__(DN_WAVES * 64) void ffn_down_kernel(
    int d, int f, int n_slots, const uint8_t *__restrict__ experts, int64_t stride, GroupSrc src,
    const int32_t *__restrict__ perm, int n_dtiles, const uint16_t *__restrict__ h_ws, float *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int g = blockIdx.x / n_dtiles;
  const int dt = blockIdx.x % n_dtiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int nb = f >> 5;
  const int srow = (nb & 3) ? nb : nb + 4;
  const int64_t plane = (int64_t)f * d / 2 + (int64_t)f * d / 32;
  const uint8_t *rec = experts + (int64_t)expert * stride;
  const uint8_t *dc = rec + 2 * plane, *ds = dc + (int64_t)d * f / 2;
  const int r0 = dt * DN_ROWS;
  const int rows_here = (d - r0) < DN_ROWS ? (d - r0) : DN_ROWS;

  // ---- stage scales of this workgroup's rows
  if ((nb & 3) == 0) {
    const int dw = nb >> 2;
    for (int idx = tid; idx < DN_ROWS * dw; idx += DN_WAVES * 64) {
      const int rr = idx / dw, cc = idx % dw;
      *(uint32_t *)(smem + rr * srow + cc * 4) = rr < rows_here ? *(const uint32_t *)(ds + (int64_t)(r0 + rr) * nb + cc * 4) : 0u;
    }
  } else {
    for (int idx = tid; idx < DN_ROWS * nb; idx += DN_WAVES * 64) {
      const int rr = idx / nb, cc = idx % nb;
      smem[rr * srow + cc] = rr < rows_here ? ds[(int64_t)(r0 + rr) * nb + cc] : 0;
    }
  }

  const bool col_ok = r < count;
  const uint16_t *hrow = h_ws + (int64_t)(start + (col_ok ? r : 0)) * 3 * f;

  const uint8_t *arow[DN_T];
  bool aok[DN_T];
#pragma unroll
  for (int t = 0; t < DN_T; ++t) {
    const int row = r0 + (wv * DN_T + t) * 16 + r;
    aok[t] = row < d;
    arow[t] = dc + (int64_t)(aok[t] ? row : 0) * (f / 2);
  }
  f32x4 acc[DN_T];
#pragma unroll
  for (int t = 0; t < DN_T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const int nsteps = (f + 127) >> 7;
  u32x4 a_nxt[DN_T];
  auto load_a = [&](int s, u32x4 *dst) {
    const int kq = (s << 7) + (q << 5);
    const bool kok = kq < f;
#pragma unroll
    for (int t = 0; t < DN_T; ++t)
      dst[t] = (aok[t] && kok) ? *(const u32x4 *)(arow[t] + (kq >> 1)) : u32x4{0u, 0u, 0u, 0u};
  };
  load_a(0, a_nxt);
  for (int s = 0; s < nsteps; ++s) {
    u32x4 a_cur[DN_T];
#pragma unroll
    for (int t = 0; t < DN_T; ++t) a_cur[t] = a_nxt[t];
    if (s + 1 < nsteps) load_a(s + 1, a_nxt);
    const int kq = (s << 7) + (q << 5);
    const bool kok = kq < f;
    float sc[DN_T];
#pragma unroll
    for (int t = 0; t < DN_T; ++t)
      sc[t] = e8m0_to_f32(smem[((wv * DN_T + t) * 16 + r) * srow + (kok ? (kq >> 5) : 0)]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 b[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[p] = (col_ok && kok) ? bits_to_bf16x8(*(const u32x4 *)(hrow + p * f + kq + 8 * j))
                               : bits_to_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int t = 0; t < DN_T; ++t) {
        const bf16x8 a = fp4x8_to_bf16(a_cur[t][j], sc[t]);
        acc[t] = mfma16x16x32(a, b[0], acc[t]);
        acc[t] = mfma16x16x32(a, b[1], acc[t]);
        acc[t] = mfma16x16x32(a, b[2], acc[t]);
      }
    }
  }

  // ---- write: lane holds y[slot of column r][rows 4*q .. 4*q+3] of each tile
  if (col_ok) {
    const int t_slot = perm[start + r];
    if (t_slot >= 0 && t_slot < n_slots) {
      float *yp = y + (int64_t)t_slot * d;
#pragma unroll
      for (int t = 0; t < DN_T; ++t) {
        const int row = r0 + (wv * DN_T + t) * 16 + 4 * q;
        if (row + 3 < d) {
          *(f32x4 *)(yp + row) = acc[t];
        } else {
          for (int i = 0; i < 4; ++i)
            if (row + i < d) yp[row + i] = acc[t][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side
static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t ffn_workspace_bytes(int64_t M, int k, int S, int d, int f, int n_experts) {
  const int64_t T = M * (k + S);
  const int64_t maxg = ffn_max_groups(M, k, S, n_experts);
  size_t b = align_up((size_t)T * 3 * f * sizeof(uint16_t), 256);
  b += align_up((size_t)maxg * sizeof(int4), 256);
  b += 256;  // n_groups
  (void)d;
  return b;
}

int64_t ffn_max_groups(int64_t M, int k, int S, int n_experts) {
  const int64_t T = M * (k + S);
  const int64_t ne = n_experts < T ? n_experts : T;
  if (M <= kGroupCols) return ne;
  return (T + kGroupCols - 1) / kGroupCols + ne;
}

int ffn_launch(const void *x, int x_bf16, int64_t M, int k, const uint8_t *experts, int64_t stride, int d, int f,
               int n_routed, int n_shared, const int32_t *offsets, const int32_t *perm, const int32_t *active,
               const int32_t *n_active, float *y, void *workspace, hipStream_t stream) {
  const int S = n_shared;
  const int kps = k + S;
  const int64_t T = M * kps;
  const int n_experts = n_routed + n_shared;
  uint8_t *ws = (uint8_t *)workspace;
  uint16_t *h_ws = (uint16_t *)ws;
  size_t off = align_up((size_t)T * 3 * f * sizeof(uint16_t), 256);
  int4 *groups = (int4 *)(ws + off);
  const int64_t maxg = ffn_max_groups(M, k, S, n_experts);
  off += align_up((size_t)maxg * sizeof(int4), 256);
  int32_t *n_groups = (int32_t *)(ws + off);

  GroupSrc src{offsets, active, n_active, nullptr, nullptr};
  if (M > kGroupCols) {
    hipLaunchKernelGGL(plan_groups_kernel, dim3(1), dim3(1024), 0, stream, offsets, active, n_active, groups,
                       n_groups);
    src.groups = groups;
    src.n_groups = n_groups;
  }
  const int n_ftiles = (f + GU_ROWS - 1) / GU_ROWS;
  const int nb_d = d / 32;
  const size_t smem_gu_scales = (size_t)2 * GU_ROWS * ((nb_d & 3) ? nb_d : nb_d + 4);
  const size_t smem_gu_red = (size_t)GU_WAVES * 32 * 64 * sizeof(float);
  const size_t smem_gu = smem_gu_scales > smem_gu_red ? smem_gu_scales : smem_gu_red;
  const int64_t grid_gu = maxg * n_ftiles;
  if (x_bf16)
    hipLaunchKernelGGL(ffn_gateup_kernel<1>, dim3((unsigned)grid_gu), dim3(GU_WAVES * 64), smem_gu, stream, x, d, f,
                       kps, (int)T, experts, stride, src, perm, n_ftiles, h_ws);
  else
    hipLaunchKernelGGL(ffn_gateup_kernel<0>, dim3((unsigned)grid_gu), dim3(GU_WAVES * 64), smem_gu, stream, x, d, f,
                       kps, (int)T, experts, stride, src, perm, n_ftiles, h_ws);
  if (hipGetLastError() != hipSuccess) return -3;
  const int n_dtiles = (d + DN_ROWS - 1) / DN_ROWS;
  const int nb_f = f / 32;
  const size_t smem_dn = (size_t)DN_ROWS * ((nb_f & 3) ? nb_f : nb_f + 4);
  hipLaunchKernelGGL(ffn_down_kernel, dim3((unsigned)(maxg * n_dtiles)), dim3(DN_WAVES * 64), smem_dn, stream, d, f,
                     (int)T, experts, stride, src, perm, n_dtiles, h_ws, y);
  if (hipGetLastError() != hipSuccess) return -3;
  return 0;
}

size_t ffn_smem_limit_ok(int d, int f) {
  const int nb_d = d / 32, nb_f = f / 32;
  const size_t a = (size_t)2 * GU_ROWS * ((nb_d & 3) ? nb_d : nb_d + 4);
  const size_t b = (size_t)DN_ROWS * ((nb_f & 3) ? nb_f : nb_f + 4);
  return a <= 65536 && b <= 65536;
}

}  // namespace moe
