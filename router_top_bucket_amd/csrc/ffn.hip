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
// product is exact and only fp32 accumulation rounds.  Every accumulation
// walks K in 128-element steps, step by step and within a step in 32-element
// MFMA slices, in ascending order: the order is fixed by d and f alone, for
// every launch shape and every M.
//
// Memory: every operand is read with buffer loads (an offset past the end
// reads zero), so lanes of empty columns, rows past f or d and K past the
// end need no branch.  Weight codes and the B operand of a step travel
// together through a ring of PF steps and are consumed in issue order, which
// is the order the vector-memory counter retires them in.
#include "common.h"
#include "launch.h"

#include <algorithm>

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
    const int4 v = src.groups[g];
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
    int v = ng;  // inclusive scan of ng over the workgroup
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o, 64);
      if (lane >= o) v += t;
    }
    if (lane == 63) wave_tot[wv] = v;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = wave_tot[w];
      if (w < wv) before += t;
      total += t;
    }
    const int excl = running + before + v - ng;
    for (int j = 0; j < ng; ++j) {
      const int rem = cnt - j * kGroupCols;
      groups[excl + j] = make_int4(e, offsets[e] + j * kGroupCols, rem < kGroupCols ? rem : kGroupCols, 0);
    }
    running += total;
    __syncthreads();
  }
  if (tid == 0) *n_groups = running;
}


// ------------------------------------------------------------------ B staging
// The B operand of a step (16 columns x 128 K, in NP bf16 parts) is loaded
// once per workgroup into an LDS ring slot and read by every wave from
// there, instead of every wave loading all of it.  Only the first MAXC
// columns are staged (no group has more slots than rows in the launch); the
// other rows of every slot are zeroed once.  A slot row is 256 bytes of data
// padded to 272 so the 16-byte fragment reads of 16 columns hit distinct
// banks.
constexpr int kBRow = 272;

template <int NP>
__device__ __forceinline__ uint32_t bslot_off(int slot, int part, int col) {
  return (uint32_t)(((slot * NP + part) * 16 + col) * kBRow);
}

__device__ __forceinline__ bf16x8 lds_b_fragment(const uint8_t *bring, uint32_t off) {
  return bits_to_bf16x8(*(const u32x4 *)(bring + off));
}

template <int NP, int PF>
__device__ __forceinline__ void zero_b_rows(uint8_t *bring, int maxc, int tid, int nthreads) {
  const int rows = PF * NP * (16 - maxc);
  for (int idx = tid; idx < rows * (kBRow / 16); idx += nthreads) {
    const int rr = idx / (kBRow / 16), cc = idx - rr * (kBRow / 16);
    const int slot_part = rr / (16 - maxc), col = maxc + rr % (16 - maxc);
    *(u32x4 *)(bring + (slot_part * 16 + col) * kBRow + cc * 16) = u32x4{0u, 0u, 0u, 0u};
  }
}

// Resident B (few columns): the group's whole B operand, MAXC columns of K
// elements in NP parts, staged once before the main loop.  Row MAXC of each
// part is zero and serves every lane whose column is past MAXC.  Each row is
// K*2 bytes followed by an 80-byte zero tail: lanes whose block lies past K
// read their fragments from the tail, and the row stride spreads the
// 16-byte reads of 8 rows over distinct banks.
constexpr int kBresTail = 80;
__host__ __device__ __forceinline__ uint32_t bres_row_bytes(int K) { return (uint32_t)(K * 2 + kBresTail); }
__host__ __device__ __forceinline__ size_t bres_bytes(int K, int maxc, int np) {
  return (size_t)np * (maxc + 1) * bres_row_bytes(K);
}

// ------------------------------------------------------------------ scales
// The E8M0 scale of a lane's 32-element block rides in the load ring with
// the codes.  With SX4 (rows of scale bytes a multiple of 16 long) one
// 16-byte load at step s = 4u brings the bytes of steps 4u..4u+3: byte
// 4*(s%4) + q of it is the scale of lane (r, q) at step s.  Otherwise one byte
// is loaded per step.  A dead step's scale is forced to 1.0: its codes read
// as zero, and the bytes past a row may be anything (0xFF would be NaN).
template <bool SX4, int NT, int PF>
struct ScaleRing {
  static_assert(!SX4 || PF % 4 == 0, "16-byte scale loads need a ring of a multiple of 4 steps");
  uint32_t soff[NT];
  u32x4 q4[SX4 ? PF / 4 : 1][NT];
  uint32_t b1[SX4 ? 1 : PF][NT];
  u32x4 cur[NT];

  // loads for step s into ring slot p (call in step order)
  __device__ __forceinline__ void issue(rsrc_t r, int s, int p, int nsteps, int smax, int q) {
    if (SX4) {
      if ((p & 3) == 0) {
        const uint32_t ks = s < nsteps ? (uint32_t)(4 * s) : kDead;
#pragma unroll
        for (int t = 0; t < NT; ++t) q4[p >> 2][t] = buf_load16(r, soff[t] + ks);
      }
    } else {
      const uint32_t ks = s < smax ? (uint32_t)(4 * s + q) : kDead;
#pragma unroll
      for (int t = 0; t < NT; ++t) b1[p][t] = buf_load1(r, soff[t] + ks);
    }
  }
  // scale of tile t at step s (slot p); call for every t before issue() refills slot p
  __device__ __forceinline__ float get(int s, int p, int t, int smax, int q) {
    uint32_t b;
    if (SX4) {
      if ((p & 3) == 0) cur[t] = q4[p >> 2][t];
      b = (cur[t][p & 3] >> (8 * q)) & 0xFFu;
    } else {
      b = b1[p][t] & 0xFFu;
    }
    return e8m0_to_f32(s < smax ? b : 127u);
  }
};

// ------------------------------------------------------------------ gate/up
// Workgroup = (group, GW*TPW*16 rows of f).  Wave w owns TPW 16-row tiles of
// W_gate and the same rows of W_up over the whole d reduction.  Lane l =
// (r = l%16, q = l/16): per step and tile it loads 16 bytes of codes = one
// 32-element MXFP4 block (row r, block q of the step).  MFMA j (0..3) of a
// step consumes elements 8j..8j+7 of each lane's block and the B fragment
// x[column r][128 s + 32 q + 8 j ..+8].
//
// x staging: piece i of a step (i < MAXC*16) is column i/16, elements
// 8*(i%16)..+8 of the step; thread t stages pieces t, t+GW*64, ...  fp32 x
// is split exactly into three bf16 parts as it is staged.
template <int XBF16, int TPW, int GW, int PF, int MAXC, bool SX4, bool BRES>
__global__ __launch_bounds__(GW * 64) void ffn_gateup_kernel(
    const void *__restrict__ x, int d, int f, int kps, int n_slots, const uint8_t *__restrict__ experts,
    int64_t stride, GroupSrc src, const int32_t *__restrict__ perm, int n_ftiles, uint16_t *__restrict__ h_ws) {
  constexpr int ROWS = GW * TPW * 16;
  constexpr int NT = 2 * TPW;  // tiles per wave: TPW gate then TPW up
  constexpr int NP = XBF16 ? 1 : 3;
  constexpr int EL = XBF16 ? 2 : 4;  // bytes per x element
  constexpr int NTH = GW * 64;
  // pieces staged per thread per step (ring mode; none in resident mode)
  constexpr int SPT = BRES ? 0 : (MAXC * 16 + NTH - 1) / NTH;
  constexpr int SPTA = SPT > 0 ? SPT : 1;  // array extent
  extern __shared__ __align__(16) uint8_t bring[];
  const int g = blockIdx.x / n_ftiles;
  const int ft = blockIdx.x - g * n_ftiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int i0 = ft * ROWS;
  const int nb = d >> 5;
  const uint32_t plane_c = (uint32_t)((int64_t)f * d / 2), plane_s = (uint32_t)((int64_t)f * d / 32);
  const uint32_t up_c = plane_c + plane_s, up_s = up_c + plane_c;
  const rsrc_t wr = make_rsrc(experts + (int64_t)expert * stride, (uint32_t)stride);
  const int M = n_slots / kps;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  const uint32_t brow = bres_row_bytes(d);
  if constexpr (BRES) {
    // stage x of the group's columns for the whole d once: 8 elements per
    // piece, MAXC columns plus the zero row, all loads issued first
    constexpr int CH = 8;  // pieces per thread per round
    const int per_col = d / 8;
    const int npieces = (MAXC + 1) * per_col;
    for (int base = 0; base < npieces; base += CH * NTH) {
      u32x4 v[CH][EL / 2];
      int pc[CH], pe[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int piece = base + c * NTH + tid;
        pc[c] = piece / per_col;
        pe[c] = (piece - pc[c] * per_col) * 8;
        uint32_t off = kOOB;
        if (piece < npieces && pc[c] < count) {
          const int t = perm[start + pc[c]];
          if (t >= 0 && t < n_slots) off = (uint32_t)(t / kps) * (uint32_t)(d * EL) + (uint32_t)(pe[c] * EL);
        }
#pragma unroll
        for (int h = 0; h < EL / 2; ++h) v[c][h] = buf_load16(xr, off + 16 * h);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (base + c * NTH + tid < npieces) {
          if (XBF16) {
            *(u32x4 *)(bring + pc[c] * brow + pe[c] * 2) = v[c][0];
          } else {
            uint32_t hi[8], mi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) split3_bf16(__uint_as_float(v[c][e >> 2][e & 3]), hi[e], mi[e], lo[e]);
            u32x4 ph, pm, pl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
              pm[e] = mi[2 * e] | (mi[2 * e + 1] << 16);
              pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
            }
            *(u32x4 *)(bring + (0 * (MAXC + 1) + pc[c]) * brow + pe[c] * 2) = ph;
            *(u32x4 *)(bring + (1 * (MAXC + 1) + pc[c]) * brow + pe[c] * 2) = pm;
            *(u32x4 *)(bring + (2 * (MAXC + 1) + pc[c]) * brow + pe[c] * 2) = pl;
          }
        }
      }
    }
    for (int idx = tid; idx < NP * (MAXC + 1) * (kBresTail / 16); idx += NTH) {
      const int row = idx / (kBresTail / 16), c = idx - row * (kBresTail / 16);
      *(u32x4 *)(bring + row * brow + d * 2 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  } else {
    zero_b_rows<NP, PF>(bring, MAXC, tid, NTH);
  }
  const int bres_r = r < MAXC ? r : MAXC;  // resident-B row of this lane's column

  // staging pieces of this thread: x row base offset (kOOB when empty) and
  // element offset within the step
  uint32_t pbase[SPTA];
  int pcol[SPTA], pel[SPTA];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int piece = tid + i * NTH;
    pcol[i] = piece >> 4;
    pel[i] = (piece & 15) * 8;
    pbase[i] = kOOB;
    if (piece < MAXC * 16 && pcol[i] < count) {
      const int t = perm[start + pcol[i]];
      if (t >= 0 && t < n_slots) pbase[i] = (uint32_t)(t / kps) * (uint32_t)(d * EL);
    }
  }
  uint32_t aoff[NT];
  ScaleRing<SX4, NT, PF> sr;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = i0 + (wv * TPW + (t % TPW)) * 16 + r;
    aoff[t] = sel_off(row < f, (t < TPW ? 0u : up_c) + (uint32_t)row * (uint32_t)(d / 2));
    sr.soff[t] = sel_off(row < f, (t < TPW ? plane_c : up_s) + (uint32_t)row * (uint32_t)nb);
  }
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (d + 127) >> 7;
  const int smax = (d - (q << 5) + 127) >> 7;  // live steps of this lane's weight block
  u32x4 ring[PF][NT];
  u32x4 xst[PF][SPTA][EL / 2];
  // Loads are consumed in the order they are issued (the vector-memory
  // counter retires in order): the codes, scales and x of step s are issued
  // together, PF-1 steps before they are used.  A dead step (past d) adds
  // kDead to every offset, which lands past every resource.
  auto issue = [&](int s, int p) {
    const int kq = (s << 7) + (q << 5);
    const uint32_t ka = s < smax ? (uint32_t)(kq >> 1) : kDead;
#pragma unroll
    for (int t = 0; t < NT; ++t) ring[p][t] = buf_load16(wr, aoff[t] + ka);
    sr.issue(wr, s, p, nsteps, smax, q);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int k = (s << 7) + pel[i];
      const uint32_t kx = k < d ? (uint32_t)(k * EL) : kDead;
#pragma unroll
      for (int h = 0; h < EL / 2; ++h) xst[p][i][h] = buf_load16(xr, pbase[i] + kx + 16 * h);
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, p);

  // The loop runs a whole number of rings: steps past the end load zeros
  // and add exact zeros, and nothing in the loop branches, so every wait on
  // the ring stays PF-1 steps deep.
  const int nsteps_pad = (nsteps + PF - 1) / PF * PF;
  for (int s0 = 0; s0 < nsteps_pad; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int s = s0 + p;
      // stage x of step s (slot p was last read at step s-PF, before the
      // previous barrier; PF >= 2)
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        if (tid + i * NTH < MAXC * 16) {
          if (XBF16) {
            *(u32x4 *)(bring + bslot_off<NP>(p, 0, pcol[i]) + pel[i] * 2) = xst[p][i][0];
          } else {
            uint32_t hi[8], mi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              split3_bf16(__uint_as_float(xst[p][i][e >> 2][e & 3]), hi[e], mi[e], lo[e]);
            u32x4 ph, pm, pl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
              pm[e] = mi[2 * e] | (mi[2 * e + 1] << 16);
              pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
            }
            *(u32x4 *)(bring + bslot_off<NP>(p, 0, pcol[i]) + pel[i] * 2) = ph;
            *(u32x4 *)(bring + bslot_off<NP>(p, 1, pcol[i]) + pel[i] * 2) = pm;
            *(u32x4 *)(bring + bslot_off<NP>(p, 2, pcol[i]) + pel[i] * 2) = pl;
          }
        }
      }
      if constexpr (!BRES) __syncthreads();
      float sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = sr.get(s, p, t, smax, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[NP];
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if constexpr (BRES)
            b[pp] = lds_b_fragment(bring, (pp * (MAXC + 1) + bres_r) * brow +
                                              (s < smax ? ((s << 7) + (q << 5) + 8 * j) * 2 : d * 2 + 16 * j));
          else
            b[pp] = lds_b_fragment(bring, bslot_off<NP>(p, pp, r) + ((q << 5) + 8 * j) * 2);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 a = fp4x8_to_bf16(ring[p][t][j], sc[t]);
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) acc[t] = mfma16x16x32(a, b[pp], acc[t]);
        }
      }
      issue(s + PF, p);
    }
  }

  // SwiGLU and the exact three-part split of h, written per slot
  if (r < count) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int row = i0 + (wv * TPW + t) * 16 + 4 * q;
      if (row < f) {
        uint32_t hi[4], mi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[t][i], uv = acc[t + TPW][i];
          split3_bf16((gv / (1.0f + expf(-gv))) * uv, hi[i], mi[i], lo[i]);
        }
        uint16_t *hp = h_ws + (int64_t)(start + r) * 3 * f + row;
        *(uint2 *)(hp) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        *(uint2 *)(hp + f) = make_uint2(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16));
        *(uint2 *)(hp + 2 * f) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Workgroup = (group, DW*TPW*16 rows of d); each wave owns TPW row tiles and
// the whole f reduction, B = the group's h in three exact bf16 parts, staged
// per step in LDS as for gate/up (piece i: part i/(MAXC*16), column
// (i/16)%MAXC, elements 8*(i%16)..+8).  Each slot's y row is written by its
// column's lanes.
template <int TPW, int DW, int PF, int MAXC, bool SX4, bool BRES>
__global__ __launch_bounds__(DW * 64) void ffn_down_kernel(
    int d, int f, int n_slots, const uint8_t *__restrict__ experts, int64_t stride, GroupSrc src,
    const int32_t *__restrict__ perm, int n_dtiles, const uint16_t *__restrict__ h_ws, float *__restrict__ y) {
  constexpr int ROWS = DW * TPW * 16;
  constexpr int NTH = DW * 64;
  constexpr int NPIECE = 3 * MAXC * 16;
  constexpr int SPT = BRES ? 0 : (NPIECE + NTH - 1) / NTH;
  constexpr int SPTA = SPT > 0 ? SPT : 1;
  extern __shared__ __align__(16) uint8_t bring[];
  const int g = blockIdx.x / n_dtiles;
  const int dt = blockIdx.x - g * n_dtiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int nb = f >> 5;
  const uint32_t plane = (uint32_t)((int64_t)f * d / 2 + (int64_t)f * d / 32);
  const uint32_t dn_c = 2 * plane, dn_s = dn_c + (uint32_t)((int64_t)d * f / 2);
  const rsrc_t wr = make_rsrc(experts + (int64_t)expert * stride, (uint32_t)stride);
  const rsrc_t hr = make_rsrc(h_ws, (uint32_t)((int64_t)n_slots * 3 * f * 2));
  const int r0 = dt * ROWS;
  const uint32_t brow = bres_row_bytes(f);
  if constexpr (BRES) {
    // stage the group's h (3 parts x MAXC columns + the zero row) for the
    // whole f once, all loads of a round issued first
    constexpr int CH = 8;
    const int per_row = f / 8;
    const int npieces = 3 * (MAXC + 1) * per_row;
    for (int base = 0; base < npieces; base += CH * NTH) {
      u32x4 v[CH];
      int prow[CH], pe[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int piece = base + c * NTH + tid;
        prow[c] = piece / per_row;  // part * (MAXC + 1) + column
        pe[c] = (piece - prow[c] * per_row) * 8;
        const int part = prow[c] / (MAXC + 1), col = prow[c] - part * (MAXC + 1);
        const uint32_t off = (piece < npieces && col < count)
                                 ? (uint32_t)(start + col) * (uint32_t)(3 * f * 2) + (uint32_t)((part * f + pe[c]) * 2)
                                 : kOOB;
        v[c] = buf_load16(hr, off);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (base + c * NTH + tid < npieces) *(u32x4 *)(bring + prow[c] * brow + pe[c] * 2) = v[c];
    }
    for (int idx = tid; idx < 3 * (MAXC + 1) * (kBresTail / 16); idx += NTH) {
      const int row = idx / (kBresTail / 16), c = idx - row * (kBresTail / 16);
      *(u32x4 *)(bring + row * brow + f * 2 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  } else {
    zero_b_rows<3, PF>(bring, MAXC, tid, NTH);
  }
  const int bres_r = r < MAXC ? r : MAXC;

  uint32_t pbase[SPTA];
  int ppart[SPTA], pcol[SPTA], pel[SPTA];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int piece = tid + i * NTH;
    ppart[i] = piece / (MAXC * 16);
    pcol[i] = (piece >> 4) % MAXC;
    pel[i] = (piece & 15) * 8;
    pbase[i] = (piece < NPIECE && pcol[i] < count)
                   ? (uint32_t)(start + pcol[i]) * (uint32_t)(3 * f * 2) + (uint32_t)(ppart[i] * f * 2)
                   : kOOB;
  }
  uint32_t aoff[TPW];
  ScaleRing<SX4, TPW, PF> sr;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = r0 + (wv * TPW + t) * 16 + r;
    aoff[t] = sel_off(row < d, dn_c + (uint32_t)row * (uint32_t)(f / 2));
    sr.soff[t] = sel_off(row < d, dn_s + (uint32_t)row * (uint32_t)nb);
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (f + 127) >> 7;
  const int smax = (f - (q << 5) + 127) >> 7;
  u32x4 ring[PF][TPW];
  u32x4 hst[PF][SPTA];
  auto issue = [&](int s, int p) {
    const int kq = (s << 7) + (q << 5);
    const uint32_t ka = s < smax ? (uint32_t)(kq >> 1) : kDead;
#pragma unroll
    for (int t = 0; t < TPW; ++t) ring[p][t] = buf_load16(wr, aoff[t] + ka);
    sr.issue(wr, s, p, nsteps, smax, q);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int k = (s << 7) + pel[i];
      hst[p][i] = buf_load16(hr, pbase[i] + (k < f ? (uint32_t)(k * 2) : kDead));
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, p);

  const int nsteps_pad = (nsteps + PF - 1) / PF * PF;  // see the gate/up kernel
  for (int s0 = 0; s0 < nsteps_pad; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int s = s0 + p;
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        if (tid + i * NTH < NPIECE) *(u32x4 *)(bring + bslot_off<3>(p, ppart[i], pcol[i]) + pel[i] * 2) = hst[p][i];
      if constexpr (!BRES) __syncthreads();
      float sc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[t] = sr.get(s, p, t, smax, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[3];
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          if constexpr (BRES)
            b[pp] = lds_b_fragment(bring, (pp * (MAXC + 1) + bres_r) * brow +
                                              (s < smax ? ((s << 7) + (q << 5) + 8 * j) * 2 : f * 2 + 16 * j));
          else
            b[pp] = lds_b_fragment(bring, bslot_off<3>(p, pp, r) + ((q << 5) + 8 * j) * 2);
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const bf16x8 a = fp4x8_to_bf16(ring[p][t][j], sc[t]);
          acc[t] = mfma16x16x32(a, b[0], acc[t]);
          acc[t] = mfma16x16x32(a, b[1], acc[t]);
          acc[t] = mfma16x16x32(a, b[2], acc[t]);
        }
      }
      issue(s + PF, p);
    }
  }

  if (r < count) {
    const int t_slot = perm[start + r];
    if (t_slot >= 0 && t_slot < n_slots) {
      float *yp = y + (int64_t)t_slot * d;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int row = r0 + (wv * TPW + t) * 16 + 4 * q;
        if (row < d) *(f32x4 *)(yp + row) = acc[t];
      }
    }
  }
}

// ------------------------------------------------------------------ host side
static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t ffn_max_groups(int64_t M, int k, int S, int n_experts) {
  const int64_t T = M * (k + S);
  const int64_t ne = n_experts < T ? n_experts : T;
  if (M <= kGroupCols) return ne;
  return (T + kGroupCols - 1) / kGroupCols + ne;
}

size_t ffn_workspace_bytes(int64_t M, int k, int S, int d, int f, int n_experts) {
  const int64_t T = M * (k + S);
  const int64_t maxg = ffn_max_groups(M, k, S, n_experts);
  size_t b = align_up((size_t)T * 3 * f * sizeof(uint16_t), 256);
  b += align_up((size_t)maxg * sizeof(int4), 256);
  b += 256;  // n_groups
  (void)d;
  return b;
}

// gfx950 gives a workgroup up to 160 KB of LDS; kernels opt in past 64 KB.
constexpr int kMaxLds = 160 * 1024;
static bool allow_lds(const void *kernel) {
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds) == hipSuccess;
}

// LDS of a launch: scale rows plus the B ring.  Every buffer resource must
// stay below 2^30 bytes (see kOOB / kDead).
static size_t gateup_smem(int d, int pf, int np, int maxc, bool bres) {
  return bres ? bres_bytes(d, maxc, np) : (size_t)pf * np * 16 * kBRow;
}
static size_t down_smem(int f, int pf, int maxc, bool bres) {
  return bres ? bres_bytes(f, maxc, 3) : (size_t)pf * 3 * 16 * kBRow;
}

bool ffn_shape_ok(int64_t M, int k, int S, int d, int f, int64_t stride) {
  const int64_t T = M * (k + S);
  const int64_t lim = (int64_t)kDead;
  (void)d;
  (void)f;
  return stride < lim &&
         M * (int64_t)d * 4 < lim && T * 3 * f * 2 < lim;
}

template <int XBF16, int TPW, int GW, int PF, int MAXC, bool SX4, bool BRES>
static int launch_gateup(const void *x, int d, int f, int kps, int T, const uint8_t *experts, int64_t stride,
                         const GroupSrc &src, const int32_t *perm, int64_t maxg, uint16_t *h_ws, hipStream_t stream) {
  constexpr int ROWS = GW * TPW * 16;
  const int n_ftiles = (f + ROWS - 1) / ROWS;
  const size_t smem = gateup_smem(d, PF, XBF16 ? 1 : 3, MAXC, BRES);
  static const bool lds_ok =
      allow_lds(reinterpret_cast<const void *>(&ffn_gateup_kernel<XBF16, TPW, GW, PF, MAXC, SX4, BRES>));
  if (!lds_ok) return -3;
  hipLaunchKernelGGL((ffn_gateup_kernel<XBF16, TPW, GW, PF, MAXC, SX4, BRES>), dim3((unsigned)(maxg * n_ftiles)), dim3(GW * 64),
                     smem, stream, x, d, f, kps, T, experts, stride, src, perm, n_ftiles, h_ws);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int TPW, int DW, int PF, int MAXC, bool SX4, bool BRES>
static int launch_down(int d, int f, int T, const uint8_t *experts, int64_t stride, const GroupSrc &src,
                       const int32_t *perm, int64_t maxg, const uint16_t *h_ws, float *y, hipStream_t stream) {
  constexpr int ROWS = DW * TPW * 16;
  const int n_dtiles = (d + ROWS - 1) / ROWS;
  const size_t smem = down_smem(f, PF, MAXC, BRES);
  static const bool lds_ok = allow_lds(reinterpret_cast<const void *>(&ffn_down_kernel<TPW, DW, PF, MAXC, SX4, BRES>));
  if (!lds_ok) return -3;
  hipLaunchKernelGGL((ffn_down_kernel<TPW, DW, PF, MAXC, SX4, BRES>), dim3((unsigned)(maxg * n_dtiles)), dim3(DW * 64), smem,
                     stream, d, f, T, experts, stride, src, perm, n_dtiles, h_ws, y);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int ffn_launch(const void *x, int x_bf16, int64_t M, int k, const uint8_t *experts, int64_t stride, int d, int f,
               int n_routed, int n_shared, const int32_t *offsets, const int32_t *perm, const int32_t *active,
               const int32_t *n_active, float *y, void *workspace, int stages, hipStream_t stream) {
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
    // the group plan lives in the workspace and serves both stages
    if (stages & kStageGateUp) {
      hipLaunchKernelGGL(plan_groups_kernel, dim3(1), dim3(1024), 0, stream, offsets, active, n_active, groups,
                         n_groups);
      if (hipGetLastError() != hipSuccess) return -3;
    }
    src.groups = groups;
    src.n_groups = n_groups;
  }
  // Launch shapes only change how many rows a wave/workgroup owns and how
  // many B columns are staged (a group never has more slots than M), never
  // the order of any reduction: every choice gives bit-identical results.
  const bool gsx4 = (d / 32) % 16 == 0, dsx4 = (f / 32) % 16 == 0;
  const int T_ = (int)T;
#define MOE_GU(XB, T, G, P, C, R)                                                                                  \
  (gsx4 ? launch_gateup<XB, T, G, P, C, true, R>(x, d, f, kps, T_, experts, stride, src, perm, maxg, h_ws, stream) \
        : launch_gateup<XB, T, G, P, C, false, R>(x, d, f, kps, T_, experts, stride, src, perm, maxg, h_ws, stream))
#define MOE_DN(T, D, P, C, R)                                                                                   \
  (dsx4 ? launch_down<T, D, P, C, true, R>(d, f, T_, experts, stride, src, perm, maxg, h_ws, y, stream) \
        : launch_down<T, D, P, C, false, R>(d, f, T_, experts, stride, src, perm, maxg, h_ws, y, stream))
  // few rows: each group's B operand (x or h) stays resident in LDS for the
  // whole reduction; more rows: B is staged step by step through a ring
  int rc = 0;
  if (stages & kStageGateUp) {
    const bool gres = gateup_smem(d, 4, x_bf16 ? 1 : 3, 4, true) <= (size_t)kMaxLds;
    if (x_bf16) {
      if (M == 1 && gres) rc = MOE_GU(1, 1, 2, 4, 1, true);
      else if (M <= 4 && gres) rc = MOE_GU(1, 1, 2, 4, 4, true);
      else if (M <= 4) rc = MOE_GU(1, 1, 4, 4, 4, false);
      else rc = MOE_GU(1, 1, 4, 4, 16, false);
    } else {
      if (M <= 4 && gres) rc = MOE_GU(0, 1, 2, 4, 4, true);
      else rc = MOE_GU(0, 1, 4, 4, 16, false);
    }
    if (rc) return rc;
  }
  if (stages & kStageDown) {
    const bool dres = down_smem(f, 4, 4, true) <= (size_t)kMaxLds;
    if (M == 1 && dres) rc = MOE_DN(2, 8, 4, 1, true);
    else if (M <= 4 && dres) rc = MOE_DN(2, 8, 4, 4, true);
    else if (M <= 4) rc = MOE_DN(2, 8, 4, 4, false);
    else rc = MOE_DN(2, 8, 4, 16, false);
  }
#undef MOE_GU
#undef MOE_DN
  return rc;
}

}  // namespace moe
