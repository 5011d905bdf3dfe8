// Expert FFN over bucketed slots: y = W_down (silu(W_gate x) * (W_up x)) with
// MXFP4 weights.  All slots of an expert are computed from one pass over its
// weights, so a multi-row block costs one weight read per distinct expert
// ("Run Kimi 3.1 locally on one GPU", section "A drafter that leaves the
// answer unchanged").
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
// scaled FP4 convert; x in bf16 is used as is and fp32 x is split exactly
// into three bf16 parts (hi + mid + lo), so every gate/up product is exact
// and only fp32 accumulation rounds.  The fp32 hidden h goes to the down pass
// as two bf16 parts (split2_bf16: |h - hi - lo| <= 2^-18 |h|), so each of its
// products is exact on those parts.  Every accumulation
// walks K in 128-element steps, step by step and within a step in 32-element
// MFMA slices, in ascending order: the order is fixed by d and f alone, for
// every launch shape and every M.
//
// Memory: every operand is read with buffer loads (an offset past the end
// reads zero), so lanes of empty columns, rows past f or d and K past the
// end need no branch.  Weight codes are streamed with non-temporal loads
// wherever a call reads an expert's codes once (every group of up to 16
// slots); the 32- and 64-wide groups of one expert re-read its codes from
// the caches and use ordinary loads.  Weight codes and the B operand of a step travel
// together through a ring of PF steps and are consumed in issue order, which
// is the order the vector-memory counter retires them in.
#include "common.h"
#include "launch.h"
#include "topk.h"

#include <algorithm>

namespace moe {

constexpr int kGroupCols = 16;
// bf16 parts of h per slot in the workspace and per slot in the down pass's
// B operand (MFMA columns)
constexpr int kHParts = 2;

// ------------------------------------------------------------------ groups
struct GroupSrc {
  const int32_t *offsets;  // direct mode: bucket offsets
  const int32_t *active;   // direct mode
  const int32_t *n_active; // direct mode
  const int4 *groups;      // plan mode: {expert, start, count, 0}
  const int32_t *n_groups; // plan mode
  const int32_t *slot_map; // null: expert e is record e; else record slot_map[e]
  int n_records;           // records at the weights base (with slot_map)
  int tiled;               // codes planes in tile order (MOE_LAYOUT_TILES), else row order
};

// Where lane (r, q) of a 16-row tile finds its 16 bytes of codes (32
// elements: block 4s+q of row `row`, row % 16 == r) inside a codes plane of
// K columns, at step 0; step s adds s * code_step().
//   row order:  row * K/2 + (4s+q) * 16
//   tile order: ((row/16) * K/32 + 4s+q) * 256 + (row%16) * 16, so the 64
//               lanes of one load read 1 KB in one piece (a permutation of
//               the same blocks: every lane gets the same bytes)
__device__ __forceinline__ uint32_t code_off(const GroupSrc &src, int row, int r, int q, int K) {
  return src.tiled ? (uint32_t)(row >> 4) * (uint32_t)(K * 8) + (uint32_t)(r * 16 + q * 256)
                   : (uint32_t)row * (uint32_t)(K / 2) + (uint32_t)(q * 16);
}
__device__ __forceinline__ uint32_t code_step(const GroupSrc &src) { return src.tiled ? 1024u : 64u; }

// Buffer resource over an expert's record.  With a slot map the record index
// is looked up, and an index outside [0, n_records) gives an empty resource:
// every load through it reads zero, none leaves the records.
__device__ __forceinline__ rsrc_t expert_rsrc(const GroupSrc &src, const uint8_t *experts, int64_t stride,
                                              int expert) {
  if (!src.slot_map) return make_rsrc(experts + (int64_t)expert * stride, (uint32_t)stride);
  const int slot = src.slot_map[expert];
  const bool ok = slot >= 0 && slot < src.n_records;
  return make_rsrc(experts + (ok ? (int64_t)slot * stride : 0), ok ? (uint32_t)stride : 0u);
}

__device__ __forceinline__ int group_count(const GroupSrc &src) { return src.groups ? *src.n_groups : *src.n_active; }

// The chip's 8 XCDs each have their own L2, and workgroup i of a launch runs
// on XCD i % 8.  Work items (group, row tile) are handed out so that XCD x
// takes a contiguous run of the real items in order: the workgroups of one
// group then share an L2 and read the group's B operand (x or h) from it
// instead of from HBM once per workgroup.  The grid holds at least the real
// item count rounded up to a multiple of 8; returns -1 for a workgroup
// without an item.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_item(int real) {
  const int x = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
  const int per = (real + kXcds - 1) / kXcds;
  const int w = x * per + j;
  return (j < per && w < real) ? w : -1;
}

__device__ __forceinline__ bool load_group(const GroupSrc &src, int g, int &expert, int &start, int &count,
                                           int maxc) {
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
  count = count < maxc ? count : maxc;
  return count > 0;
}

// One-row layer calls in one launch (route mode): the router logits of the
// row are the input, and group g of the launch is the row's g-th expert in
// bucket order: its k routed experts by ascending id (ids are below E), then
// the S shared ones.  A workgroup of a shared expert knows it at once; one
// of a routed expert ranks the logits in its first wave (topk_row, the top-k
// kernel's code, so the set and its rank order are the top-k kernel's) and
// takes the id at ascending position g.  The workgroup of item 0 also writes
// what the top-k and bucket kernels would (ids, weights, offsets, perm,
// active, n_active, dev_error: the same code, the same bits); the down pass
// and the combine read them after this launch.  Every thread of the
// workgroup calls this.  `lists`: at least topk_wave_lds(16) bytes of LDS,
// free until the function returns.
__device__ int route_one_row(const RouteArgs &ra, int g, bool writer, uint8_t *lists, int *bcast) {
  if (g >= ra.k) return ra.E + (g - ra.k);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int32_t id;
    float wt;
    // only the writer stores the weights; the others need the ids alone
    topk_row_any<16>(ra.logits, ra.E, ra.k, (uint64_t(*)[64])lists, lane, id, wt, writer);
    int pos = 0;  // ascending position of this lane's id among the k (distinct) ids
    for (int i = 0; i < ra.k; ++i) pos += __builtin_amdgcn_readlane(id, i) < id;
    const uint64_t hit = __ballot(lane < ra.k && pos == g);
    const int e = __builtin_amdgcn_readlane(id, (int)__ffsll((unsigned long long)hit) - 1);
    if (lane == 0) *bcast = e;
    if (writer) {
      if (lane < ra.k) {
        ra.ids[lane] = id;
        ra.w[lane] = wt;
      }
      bucket_one_row(id, lane, ra.E, ra.k, ra.S, ra.offsets, ra.perm, ra.active, ra.n_active, ra.dev_error);
    }
  }
  lds_barrier();  // the expert is in LDS, and the first wave is done with the lists
  return *bcast;
}

// Many rows: one workgroup cuts every active expert's segment into groups
// and sorts them into three lists by width (without `wide`, every segment is
// cut into narrow groups of 16, all in list 0).  An expert with at most 16 slots
// is one narrow group; a longer segment is cut into groups of 64 slots, and
// its remainder (if any) is a narrow (<= 16), a 32-wide (17..32) or a 64-wide
// (33..63) group.  Lists: class 0 narrow, 1 up to 32 slots, 2 up to 64.
constexpr int kWideCols = 64;
constexpr int kGroupClasses = 3;

__device__ __forceinline__ int group_class(int cnt) { return cnt <= kGroupCols ? 0 : (cnt <= 32 ? 1 : 2); }

__global__ __launch_bounds__(1024) void plan_groups_kernel(const int32_t *offsets, const int32_t *active,
                                                           const int32_t *n_active, int4 *groups0, int4 *groups1,
                                                           int4 *groups2, int32_t *n_groups, int wide) {
  __shared__ int32_t wave_tot[kGroupClasses][16];
  const int na = *n_active;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int4 *const lists[kGroupClasses] = {groups0, groups1, groups2};
  int running[kGroupClasses] = {0, 0, 0};  // groups emitted by earlier passes, per class
  for (int base = 0; base < na; base += 1024) {
    const int i = base + tid;
    int cnt = 0, e = 0;
    int ng[kGroupClasses] = {0, 0, 0};
    if (i < na) {
      e = active[i];
      cnt = offsets[e + 1] - offsets[e];
      if (!wide) {
        ng[0] = (cnt + kGroupCols - 1) / kGroupCols;
      } else if (cnt <= kGroupCols) {
        ng[0] = cnt > 0 ? 1 : 0;
      } else {
        const int full = cnt / kWideCols, rem = cnt - full * kWideCols;
        ng[2] = full;
        if (rem > 0) ++ng[group_class(rem)];
      }
    }
    int excl[kGroupClasses], total[kGroupClasses];
#pragma unroll
    for (int c = 0; c < kGroupClasses; ++c) {
      int v = ng[c];  // inclusive scan over the workgroup
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
      }
      if (lane == 63) wave_tot[c][wv] = v;
      __syncthreads();
      int before = 0, tot = 0;
      for (int w = 0; w < 16; ++w) {
        const int t = wave_tot[c][w];
        if (w < wv) before += t;
        tot += t;
      }
      excl[c] = running[c] + before + v - ng[c];
      total[c] = tot;
      __syncthreads();
    }
    if (i < na && cnt > 0) {
      const int o = offsets[e];
      if (!wide) {
        for (int jj = 0; jj < ng[0]; ++jj) {
          const int rem = cnt - jj * kGroupCols;
          lists[0][excl[0] + jj] = make_int4(e, o + jj * kGroupCols, rem < kGroupCols ? rem : kGroupCols, 0);
        }
      } else if (cnt <= kGroupCols) {
        lists[0][excl[0]] = make_int4(e, o, cnt, 0);
      } else {
        const int full = cnt / kWideCols, rem = cnt - full * kWideCols;
        for (int j = 0; j < full; ++j) lists[2][excl[2] + j] = make_int4(e, o + j * kWideCols, kWideCols, 0);
        if (rem > 0) {
          const int c = group_class(rem);
          lists[c][excl[c] + (c == 2 ? full : 0)] = make_int4(e, o + full * kWideCols, rem, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kGroupClasses; ++c) running[c] += total[c];
  }
  if (tid < kGroupClasses) n_groups[tid] = running[tid];
}

// ------------------------------------------------------------------ B staging
// Ring mode: the B operand of a step (a 128-element segment of every B row)
// is loaded once per workgroup into an LDS ring slot and read by every wave
// from there.  A slot row is 256 bytes of data padded to 272, so the 16-byte
// fragment reads of 16 rows hit distinct banks.
constexpr int kBRow = 272;

__device__ __forceinline__ bf16x8 lds_b_fragment(const uint8_t *lds, uint32_t off) {
  return bits_to_bf16x8(*(const u32x4 *)(lds + off));
}

// Resident mode (few rows): every B row for the whole reduction, staged once
// before the main loop.  Each row is K*2 bytes followed by an 80-byte zero
// tail: lanes whose 32-element block lies past K read their fragments from
// the tail, and the stride spreads the 16-byte reads of 8 rows over distinct
// banks.
constexpr int kBresTail = 80;
__host__ __device__ __forceinline__ uint32_t bres_row_bytes(int K) { return (uint32_t)(K * 2 + kBresTail); }

// Epilogue exchange areas follow the B area in LDS, 16-byte aligned, then a
// small dummy area: a staging load whose piece lies past the data is still
// stored, there, so that every load is consumed on every path.  (A load left
// unconsumed on some path makes the compiler assume it may still be pending
// when the main loop starts, and wait for all loads in flight at every
// iteration, which drains the prefetch ring.)
__host__ __device__ __forceinline__ size_t lds_align16(size_t v) { return (v + 15) & ~(size_t)15; }

// Scale rows staged in LDS: a row's K/32 E8M0 bytes followed by a zero tail
// that the steps past K read (lanes of blocks past the end, padded steps).
constexpr int kScTail = 48;
__host__ __device__ __forceinline__ int sc_pitch(int K) { return (int)lds_align16((size_t)(K / 32 + kScTail)); }

// Gate/up LDS: the scale rows of both matrices (2*ROWS), B (resident: NP*MAXC
// rows; ring: PF slots of NP*16 rows), the W_up tiles (ROWS x 17 floats),
// then the dummy area.
__host__ __device__ __forceinline__ size_t gateup_b_off(int d, int rows) { return lds_align16((size_t)2 * rows * sc_pitch(d)); }
__host__ __device__ __forceinline__ size_t gateup_b_bytes(int d, int pf, int np, int maxc, bool bres) {
  return bres ? (size_t)np * maxc * bres_row_bytes(d) : (size_t)pf * np * 16 * kBRow;
}
__host__ __device__ __forceinline__ size_t gateup_e_off(int d, int pf, int np, int maxc, bool bres, int rows) {
  return lds_align16(gateup_b_off(d, rows) + gateup_b_bytes(d, pf, np, maxc, bres));
}
__host__ __device__ __forceinline__ size_t gateup_dummy_off(int d, int pf, int np, int maxc, bool bres, int rows) {
  return lds_align16(gateup_e_off(d, pf, np, maxc, bres, rows) + (size_t)rows * 17 * sizeof(float));
}
__host__ __device__ __forceinline__ size_t gateup_lds_bytes(int d, int pf, int np, int maxc, bool bres, int rows) {
  return gateup_dummy_off(d, pf, np, maxc, bres, rows) + 16 * 3;
}
// Down LDS: the scale rows (ROWS; none when the scales travel with the ring
// loads, scr), then B (resident: 3*MAXC rows; ring: PF slots of 3*MAXC
// rows), whose space the per-(row, column) part sums of YC columns at a time
// (YC columns of ROWS + 4 floats, see down_yc) reuse once the main loop is
// done, then the dummy area.
__host__ __device__ __forceinline__ size_t down_b_off(int f, int rows, bool scr = false) {
  return scr ? 0 : lds_align16((size_t)rows * sc_pitch(f));
}
__host__ __device__ __forceinline__ size_t down_b_bytes(int f, int pf, int maxc, bool bres) {
  return bres ? (size_t)kHParts * maxc * bres_row_bytes(f) : (size_t)pf * kHParts * maxc * kBRow;
}
__host__ __device__ __forceinline__ size_t down_y_off(int f, int pf, int maxc, bool bres, int rows, bool scr = false) {
  return down_b_off(f, rows, scr);
}
// Columns of the epilogue's per-(row, column) sums held at a time: all of
// them for up to 16 slots (or a resident B), else as many whole 16-slot
// blocks (16 kHParts columns) as the ring slots' bytes hold.
__host__ __device__ constexpr int down_yc(int pf, int maxc, bool bres, int rows) {
  constexpr int blk = 16 * kHParts;  // the columns of 16 slots
  const int nc = kHParts * maxc;
  const int avail = (int)((size_t)pf * nc * kBRow / ((size_t)(rows + 4) * 4));
  const int yc = avail / blk * blk;
  return (bres || nc <= blk) ? nc : (yc < blk ? blk : (yc > nc ? nc : yc));
}
__host__ __device__ __forceinline__ size_t down_dummy_off(int f, int pf, int maxc, bool bres, int rows,
                                                          bool scr = false) {
  const int yc = down_yc(pf, maxc, bres, rows);
  const size_t b = down_b_bytes(f, pf, maxc, bres), y = (size_t)yc * (rows + 4) * sizeof(float);
  return lds_align16(down_b_off(f, rows, scr) + (b > y ? b : y));
}
__host__ __device__ __forceinline__ size_t down_lds_bytes(int f, int pf, int maxc, bool bres, int rows,
                                                          bool scr = false) {
  return down_dummy_off(f, pf, maxc, bres, rows, scr) + 16;
}

// ------------------------------------------------------------------ scales
// Every scale byte a workgroup needs is copied into LDS once, before the main
// loop: the scales of a run of consecutive weight rows are one contiguous span
// of the scales plane, so the copy is a handful of wide coalesced loads.
// (Loading them through the ring instead adds a small request per row every
// few steps, and the streaming loop is bound by the number of requests.)
// At step s lane (r, q) reads byte 4s + q of its row: the scale of its block.
//
// ScaleStage: rows [0, nrows) of `lds_sc` (pitch sc_pitch(K)) get the nb =
// K/32 scale bytes of global weight rows row0.. (scales plane at `plane`);
// rows at or past `rows_valid` and every tail get zeros.  begin() issues the
// loads of the first round of pieces, end() stores them and stages any
// further rounds (loads before stores), so that a kernel can issue begin()
// before its ring prefill and let one wait cover both.  Every load is stored
// (to `dummy` when out of range).  STREAM: wide loads carry the non-temporal
// hint (the ring-mode kernels; measured faster there, slower at 1 row).
template <bool W16, bool STREAM = false>
struct ScaleStage {
  static constexpr int CH = W16 ? 4 : 8;  // pieces per thread per round
  u32x4 v16[W16 ? CH : 1];
  uint32_t v1[W16 ? 1 : CH];
  int pr[CH], pc[CH];
  int per_row, npieces;

  __device__ __forceinline__ void load_round(rsrc_t wr, uint32_t plane, int row0, int rows_valid, int nb, int base,
                                             int tid, int nth) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int piece = base + c * nth + tid;
      pr[c] = piece / per_row;
      pc[c] = piece - pr[c] * per_row;
      const bool ok = piece < npieces && pr[c] < rows_valid;
      if (W16) {
        const uint32_t o = ok ? plane + (uint32_t)(row0 + pr[c]) * (uint32_t)nb + 16u * pc[c] : kOOB;
        v16[c] = STREAM ? buf_load16_stream(wr, o) : buf_load16(wr, o);
      } else
        v1[c] = buf_load1(wr, ok ? plane + (uint32_t)(row0 + pr[c]) * (uint32_t)nb + (uint32_t)pc[c] : kOOB);
    }
  }
  __device__ __forceinline__ void store_round(uint8_t *lds_sc, int sp, uint32_t dummy_off, uint8_t *lds, int base,
                                              int tid, int nth) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool live = base + c * nth + tid < npieces;
      if (W16)
        *(u32x4 *)(live ? lds_sc + pr[c] * sp + 16 * pc[c] : lds + dummy_off) = v16[c];
      else
        *(live ? lds_sc + pr[c] * sp + pc[c] : lds + dummy_off) = (uint8_t)v1[c];
    }
  }
  __device__ __forceinline__ void begin(rsrc_t wr, uint32_t plane, int row0, int rows_valid, int nrows, int K, int tid,
                                        int nth) {
    const int nb = K >> 5;
    per_row = W16 ? nb >> 4 : nb;  // W16: nb is a multiple of 16, 16-byte pieces
    npieces = nrows * per_row;
    load_round(wr, plane, row0, rows_valid, nb, 0, tid, nth);
  }
  __device__ __forceinline__ void end(rsrc_t wr, uint32_t plane, int row0, int rows_valid, int nrows, int K,
                                      uint8_t *lds_sc, uint32_t dummy_off, uint8_t *lds, int tid, int nth) {
    const int nb = K >> 5, sp = sc_pitch(K);
    store_round(lds_sc, sp, dummy_off, lds, 0, tid, nth);
    for (int base = CH * nth; base < npieces; base += CH * nth) {
      load_round(wr, plane, row0, rows_valid, nb, base, tid, nth);
      store_round(lds_sc, sp, dummy_off, lds, base, tid, nth);
    }
    // zero tails: bytes [nb, sp) of every row
    const int tail16 = (sp - (nb & ~15)) >> 4;  // 16-byte pieces from the last aligned offset
    for (int idx = tid; idx < nrows * tail16; idx += nth) {
      const int row = idx / tail16, c = idx - row * tail16;
      uint8_t *pt = lds_sc + row * sp + (nb & ~15) + 16 * c;
      if (c == 0 && (nb & 15)) {
        for (int k = nb & 15; k < 16; ++k) pt[k] = 0;
      } else {
        *(u32x4 *)pt = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
};

// Scale of lane (r, q)'s block at step s, from its LDS row.
__device__ __forceinline__ float lds_scale(const uint8_t *row, int s, int q) {
  return __builtin_ldexpf(1.0f, (int)row[4 * s + q] - 127);
}

// ------------------------------------------------------------------ gate/up
// Workgroup = (group, ROWS rows of f).  PAIR: each of the GW waves owns TPW
// 16-row tiles of W_gate and the same rows of W_up (ROWS = GW * TPW * 16),
// and forms SwiGLU itself.  Otherwise the first GW/2 waves own TPW tiles of
// W_gate and the other GW/2 the same rows of W_up (ROWS = GW/2 * TPW * 16),
// and the W_up waves hand their tiles over through LDS.  Each tile covers the
// whole d reduction.  Lane l = (r = l%16, q = l/16): per
// step and tile it loads 16 bytes of codes = one 32-element MXFP4 block (row
// r, block q of the step).  MFMA j (0..3) of a step consumes elements
// 8j..8j+7 of each lane's block and the B fragment x[column r][128 s + 32 q +
// 8 j ..+8].  Column r is slot r of the group.  In resident mode the lanes of
// columns past the group's slots read column 0: an MFMA output column
// depends only on its own B column, and those columns are never stored.
//
// Epilogue: h = silu(g) * u for every slot, split into kHParts bf16 parts
// (split2_bf16).
//
// x staging (ring mode): piece i of a step (i < MAXC*16) is column i/16,
// elements 8*(i%16)..+8 of the step; thread t stages pieces t, t+GW*64, ...
// fp32 x is split exactly into three bf16 parts as it is staged.
//
// ROUTE (one row, resident B): the groups come from the router logits
// (route_one_row) instead of the bucketing arrays, which this launch writes.
template <int XBF16, int TPW, int GW, int PF, int MAXC, bool SX4, bool BRES, bool PAIR, bool ROUTE = false>
__global__ __launch_bounds__(GW * 64) void ffn_gateup_kernel(
    const void *__restrict__ x, int d, int f, int kps, int n_slots, const uint8_t *__restrict__ experts,
    int64_t stride, GroupSrc src, const int32_t *__restrict__ perm, int n_ftiles, uint16_t *__restrict__ h_ws,
    RouteArgs ra) {
  static_assert(PAIR || GW % 2 == 0, "gate and up waves come in pairs");
  static_assert(!ROUTE || BRES, "route mode stages x once (one row)");
  constexpr int HW = PAIR ? GW : GW / 2;  // waves per row group
  constexpr int ROWS = HW * TPW * 16;
  constexpr int NT = PAIR ? 2 * TPW : TPW;  // tiles per wave
  constexpr int NP = XBF16 ? 1 : 3;
  constexpr int EL = XBF16 ? 2 : 4;  // bytes per x element
  constexpr int NTH = GW * 64;
  // pieces staged per thread per step (ring mode; none in resident mode)
  constexpr int SPT = BRES ? 0 : (MAXC * 16 + NTH - 1) / NTH;
  constexpr int SPTA = SPT > 0 ? SPT : 1;  // array extent
  extern __shared__ __align__(16) uint8_t lds[];
  const int item = xcd_item((ROUTE ? ra.k + ra.S : group_count(src)) * n_ftiles);
  if (item < 0) return;
  const int g = item / n_ftiles;
  const int ft = item - g * n_ftiles;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M = n_slots / kps;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  const uint32_t brow = bres_row_bytes(d);
  const uint32_t dummy = (uint32_t)gateup_dummy_off(d, PF, NP, MAXC, BRES, ROWS);
  uint8_t *const bmem = lds + gateup_b_off(d, ROWS);  // B area (after the scale rows)

  // Resident B: x of the group's `cnt` columns (x row offsets xb, kOOB past
  // the group) for the whole d, 8 elements per piece, all loads of a round
  // issued before its LDS writes; threads t0 .. t0 + nthr - 1 take part.
  auto stage_x = [&](int cnt, const uint32_t (&xb)[MAXC], int t0, int nthr) {
    constexpr int CH = 8;  // pieces per thread per round
    const int per_col = d / 8;
    const int npieces = cnt * per_col;
    for (int base = 0; base < npieces; base += CH * nthr) {
      u32x4 v[CH][EL / 2];
      int pc[CH], pe[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int piece = base + c * nthr + t0;
        pc[c] = piece / per_col;
        pe[c] = (piece - pc[c] * per_col) * 8;
        uint32_t xrow = xb[0];
#pragma unroll
        for (int cc = 1; cc < MAXC; ++cc) xrow = pc[c] == cc ? xb[cc] : xrow;
        const uint32_t off = piece < npieces ? xrow + (uint32_t)(pe[c] * EL) : kOOB;
#pragma unroll
        for (int h = 0; h < EL / 2; ++h) v[c][h] = buf_load16(xr, off + 16 * h);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const bool live = base + c * nthr + t0 < npieces;
        if (XBF16) {
          *(u32x4 *)(live ? bmem + pc[c] * brow + pe[c] * 2 : lds + dummy) = v[c][0];
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
          *(u32x4 *)(live ? bmem + (0 * MAXC + pc[c]) * brow + pe[c] * 2 : lds + dummy) = ph;
          *(u32x4 *)(live ? bmem + (1 * MAXC + pc[c]) * brow + pe[c] * 2 : lds + dummy + 16) = pm;
          *(u32x4 *)(live ? bmem + (2 * MAXC + pc[c]) * brow + pe[c] * 2 : lds + dummy + 32) = pl;
        }
      }
    }
    for (int idx = t0; idx < NP * MAXC * (kBresTail / 16); idx += nthr) {
      const int row = idx / (kBresTail / 16), c = idx - row * (kBresTail / 16);
      *(u32x4 *)(bmem + row * brow + d * 2 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  int expert, start, count;
  // route mode, a routed group: x (the one row, row 0) does not depend on
  // the ranking, so the other waves stage it while the first wave ranks,
  // where the B area lies past the ranking's LDS
  bool x_staged = false;
  if constexpr (ROUTE) {
    __shared__ int route_bcast;
    x_staged = g < ra.k && gateup_b_off(d, ROWS) >= topk_wave_lds(16);
    if (x_staged && tid >= 64) {
      uint32_t xb[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) xb[c] = c == 0 ? 0u : kOOB;
      stage_x(1, xb, tid - 64, NTH - 64);
    }
    expert = route_one_row(ra, g, item == 0, lds, &route_bcast);  // its barrier publishes x too
    start = g;  // one slot per expert: bucket position g
    count = 1;
  } else {
    if (!load_group(src, g, expert, start, count, MAXC)) return;
  }

  const int r = lane & 15, q = lane >> 4;
  const int mat = PAIR ? 0 : (wv >= HW ? 1 : 0);  // 0: W_gate, 1: W_up (split layout)
  const int rw = wv - mat * HW;                    // row-tile group of this wave
  const int i0 = ft * ROWS;
  const uint32_t plane_c = (uint32_t)((int64_t)f * d / 2), plane_s = (uint32_t)((int64_t)f * d / 32);
  const rsrc_t wr = expert_rsrc(src, experts, stride, expert);
  const int bcol = r < count ? r : 0;  // resident-B column read by this lane

  // staging pieces of this thread: x row base offset (kOOB when empty) and
  // element offset within the step
  uint32_t pbase[SPTA];
  int pcol[SPTA], pel[SPTA];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int piece = tid + i * NTH;
    pcol[i] = piece >> 4;
    pel[i] = (piece & 15) * 8;
    const int t = perm[start + (pcol[i] < count ? pcol[i] : count - 1)];
    pbase[i] = (piece < MAXC * 16 && pcol[i] < count && t >= 0 && t < n_slots) ? (uint32_t)(t / kps) * (uint32_t)(d * EL)
                                                                                 : kOOB;
  }
  uint32_t aoff[NT];
  const uint8_t *srow[NT];  // this lane's LDS scale row per tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tm = PAIR ? t / TPW : mat;  // matrix of tile t
    const int lrow = (rw * TPW + t % TPW) * 16 + r;
    const int row = i0 + lrow;
    aoff[t] = sel_off(row < f, (tm ? plane_c + plane_s : 0u) + code_off(src, row, r, q, d));
    srow[t] = lds + (tm * ROWS + lrow) * sc_pitch(d);
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
  const uint32_t cstep = code_step(src);
  auto issue = [&](int s, int p) {
    const uint32_t ka = s < smax ? (uint32_t)s * cstep : kDead;
#pragma unroll
    for (int t = 0; t < NT; ++t) ring[p][t] = buf_load16_stream(wr, aoff[t] + ka);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int k = (s << 7) + pel[i];
      const uint32_t kx = k < d ? (uint32_t)(k * EL) : kDead;
#pragma unroll
      for (int h = 0; h < EL / 2; ++h) xst[p][i][h] = buf_load16(xr, pbase[i] + kx + 16 * h);
    }
  };
  // the scale staging loads go first, then the ring prefill; one wait covers
  // both (ring mode: with every load arrived the compiler sees the same loads
  // in flight at every loop iteration, instead of keeping the prefill's issue
  // order in mind at the loop head and waiting far deeper than the ring needs)
  const int rv = f - i0 < ROWS ? f - i0 : ROWS;
  ScaleStage<SX4, !BRES> sg, su;
  sg.begin(wr, plane_c, i0, rv, ROWS, d, tid, NTH);
  su.begin(wr, 2 * plane_c + plane_s, i0, rv, ROWS, d, tid, NTH);
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, p);
  asm volatile("" ::: "memory");
  if constexpr (!BRES) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  asm volatile("" ::: "memory");
  sg.end(wr, plane_c, i0, rv, ROWS, d, lds, dummy, lds, tid, NTH);
  su.end(wr, 2 * plane_c + plane_s, i0, rv, ROWS, d, lds + ROWS * sc_pitch(d), dummy, lds, tid, NTH);
  if constexpr (BRES) {
    if (!x_staged) {
      // the x row of each column, read from perm once, up front
      uint32_t xb[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        // route mode: the one row's slots (perm is being written by this launch)
        const int t = ROUTE ? 0 : perm[start + (c < count ? c : count - 1)];
        xb[c] = (c < count && t >= 0 && t < n_slots) ? (uint32_t)(t / kps) * (uint32_t)(d * EL) : kOOB;
      }
      stage_x(count, xb, tid, NTH);
    }
    lds_barrier();  // the scale rows (and x) are in LDS
  } else if constexpr (MAXC < 16) {
    // rows of columns >= MAXC are never staged: zero them once
    const int zrows = PF * NP * (16 - MAXC);
    for (int idx = tid; idx < zrows * (kBRow / 16); idx += NTH) {
      const int rr = idx / (kBRow / 16), cc = idx - rr * (kBRow / 16);
      const int slot_part = rr / (16 - MAXC), col = MAXC + rr % (16 - MAXC);
      *(u32x4 *)(bmem + (slot_part * 16 + col) * kBRow + cc * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }

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
        {
          const bool live = tid + i * NTH < MAXC * 16;
          uint8_t *dst = live ? bmem + ((p * NP) * 16 + pcol[i]) * kBRow + pel[i] * 2 : lds + dummy;
          const uint32_t pstep = live ? 16 * kBRow : 16;
          if (XBF16) {
            *(u32x4 *)dst = xst[p][i][0];
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
            *(u32x4 *)dst = ph;
            *(u32x4 *)(dst + pstep) = pm;
            *(u32x4 *)(dst + 2 * pstep) = pl;
          }
        }
      }
      if constexpr (!BRES) lds_barrier();
      float sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = lds_scale(srow[t], s, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[NP];
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if constexpr (BRES)
            b[pp] = lds_b_fragment(bmem, (pp * MAXC + bcol) * brow +
                                            (s < smax ? ((s << 7) + (q << 5) + 8 * j) * 2 : d * 2 + 16 * j));
          else
            b[pp] = lds_b_fragment(bmem, ((p * NP + pp) * 16 + r) * kBRow + ((q << 5) + 8 * j) * 2);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 a = fp4x8_to_bf16(ring[p][t][j], sc[t]);
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) acc[t] = mfma16x16x32(a, b[pp], acc[t]);
        }
      }
      issue(s + PF, p);
      // keep the refill here: the scheduler would otherwise sink it past the
      // next steps' waits and drain the ring once per unrolled window
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // SwiGLU: split layout: the W_up waves hand their tiles to the W_gate
  // waves through LDS; paired layout: both are in the wave already
  float *ut = (float *)(lds + gateup_e_off(d, PF, NP, MAXC, BRES, ROWS));
  if (!PAIR) {
    if (mat) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) ut[((rw * TPW + t) * 16 + 4 * q + i) * 17 + r] = acc[t][i];
    }
    lds_barrier();
  }
  if (!mat && r < count) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int lrow = (rw * TPW + t) * 16 + 4 * q;
      const int row = i0 + lrow;
      if (row < f) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[t][i], uv = PAIR ? acc[(t + TPW) % NT][i] : ut[(lrow + i) * 17 + r];
          split2_bf16((gv / (1.0f + expf(-gv))) * uv, hi[i], lo[i]);
        }
        uint16_t *hp = h_ws + (int64_t)(start + r) * kHParts * f + row;
        *(uint2 *)(hp) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        *(uint2 *)(hp + f) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      }
    }
  }
}

// ------------------------------------------------------------------ wide gate/up
// Groups of up to 16*NCB slots (an expert with many rows): the arithmetic of
// ffn_gateup_kernel (same decode, same K order, same parts), with NCB
// 16-column blocks per group so that each decoded weight fragment feeds NCB
// MFMAs per part.  Each of the GW waves owns two 16-row tiles of W_gate and
// the same rows of W_up (ROWS = 32 GW) and forms SwiGLU itself.  The B
// operand of a step (16*NCB columns, columns past the group's slots staged as
// zeros) goes through an LDS ring of PF slots as in ring mode.  Scales travel
// with the loads instead of being staged: every 4 steps lane (r, q) of a tile
// loads the dword of its row that holds the 4 block scales of step 4j + q,
// and at step 4j + u a bpermute from lane (r, u) hands lane (r, q) byte q.
// Needs d % 128 == 0 (dword-aligned scale rows).
//
// DMA (bf16 x): x goes straight into its ring slot by LDS DMA, as the down
// kernel's B (256-byte rows, chunk c of column j at position c ^ (j % 16);
// slot (s-1) % PF refilled with step s+PF-1 after step s's barrier; step s
// waits for its own DMA loads by count).  Bit-identical to register staging.
template <int XBF16, int GW, int PF, int NCB, bool DMA = false>
__global__ __launch_bounds__(GW * 64) void ffn_gateup_wide_kernel(
    const void *__restrict__ x, int d, int f, int kps, int n_slots, const uint8_t *__restrict__ experts,
    int64_t stride, GroupSrc src, const int32_t *__restrict__ perm, int n_ftiles, uint16_t *__restrict__ h_ws) {
  static_assert(4 % PF == 0 && PF >= 2, "ring depth divides the 4-step scale group");
  constexpr int NT = 4;  // W_gate rows +0, +16; W_up rows +0, +16
  constexpr int ROWS = GW * 32;
  constexpr int MAXC = 16 * NCB;
  constexpr int NP = XBF16 ? 1 : 3;
  constexpr int EL = XBF16 ? 2 : 4;
  constexpr int NTH = GW * 64;
  constexpr int SPT = (MAXC * 16 + NTH - 1) / NTH;
  constexpr uint32_t SLOT = (uint32_t)NP * MAXC * kBRow;
  static_assert(!DMA || (XBF16 && (MAXC * 16) % NTH == 0), "LDS DMA: bf16 x, whole 1 KB pieces per wave");
  constexpr uint32_t SLOTD = (uint32_t)MAXC * 256u;  // DMA: one ring slot, 256-byte rows
  extern __shared__ __align__(16) uint8_t lds[];
  const int item = xcd_item(group_count(src) * n_ftiles);
  if (item < 0) return;
  const int g = item / n_ftiles;
  const int ft = item - g * n_ftiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count, MAXC)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int i0 = ft * ROWS;
  const int nb = d >> 5;
  const uint32_t plane_c = (uint32_t)((int64_t)f * d / 2), plane_s = (uint32_t)((int64_t)f * d / 32);
  const rsrc_t wr = expert_rsrc(src, experts, stride, expert);
  const int M = n_slots / kps;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * d * EL));
  const uint32_t dummy = PF * SLOT;

  uint32_t pbase[SPT];
  int pcol[SPT], pel[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int piece = tid + i * NTH;
    pcol[i] = piece >> 4;
    // DMA: the chunk stored at position piece % 16 of column pcol
    pel[i] = DMA ? ((piece & 15) ^ (pcol[i] & 15)) * 8 : (piece & 15) * 8;
    const int t = perm[start + (pcol[i] < count ? pcol[i] : count - 1)];
    pbase[i] = (piece < MAXC * 16 && pcol[i] < count && t >= 0 && t < n_slots)
                   ? (uint32_t)(t / kps) * (uint32_t)(d * EL)
                   : kOOB;
  }
  uint32_t aoff[NT], soff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tm = t >> 1;
    const int row = i0 + wv * 32 + (t & 1) * 16 + r;
    aoff[t] = sel_off(row < f, (tm ? plane_c + plane_s : 0u) + code_off(src, row, r, q, d));
    soff[t] = sel_off(row < f, (tm ? 2 * plane_c + plane_s : plane_c) + (uint32_t)row * (uint32_t)nb + 4u * q);
  }
  f32x4 acc[NT][NCB];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (d + 127) >> 7;
  const int smax = (d - (q << 5) + 127) >> 7;
  const int ngroups = (nsteps + 3) >> 2;
  u32x4 ring[PF][NT];
  u32x4 xst[PF][DMA ? 1 : SPT][EL / 2];
  uint32_t sc_cur[NT], sc_nxt[NT];
  const uint32_t cstep = code_step(src);
  auto issue = [&](int s, int p) {
    const uint32_t ka = s < smax ? (uint32_t)s * cstep : kDead;
#pragma unroll
    for (int t = 0; t < NT; ++t) ring[p][t] = buf_load16(wr, aoff[t] + ka);
    if constexpr (!DMA) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int k = (s << 7) + pel[i];
        const uint32_t kx = k < d ? (uint32_t)(k * EL) : kDead;
#pragma unroll
        for (int h = 0; h < EL / 2; ++h) xst[p][i][h] = buf_load16(xr, pbase[i] + kx + 16 * h);
      }
    }
  };
  // DMA: x of step s into ring slot p, one 1 KB piece per wave instruction
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  auto dma_x = [&](int s, int p) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int k = (s << 7) + pel[i];
      buf_load16_lds(xr, pbase[i] + (k < d ? (uint32_t)(k * EL) : kDead), lds + p * SLOTD + (uint32_t)(i * NTH + wvu * 64) * 16u);
    }
  };
  // lane q loads the scale dword of step 4j + q; the dword of a padding step
  // (past d) would lie past the row's d/32 scale bytes, in the next row or
  // plane, where a 0xFF byte would make the scale infinite and its zero codes
  // NaN, so such lanes read past the resource (zero bytes) instead
  auto load_sc = [&](int j, uint32_t (&sc)[NT]) {
    const uint32_t js = (j < ngroups && 4 * j + q < nsteps) ? 16u * (uint32_t)j : kDead;
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[t] = buf_load4(wr, soff[t] + js);
  };

  load_sc(0, sc_cur);
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, p);
  if constexpr (DMA) {
#pragma unroll
    for (int p = 0; p < PF - 1; ++p) dma_x(p, p);
  }
  // start the loop with nothing in flight (the waits inside it are then the
  // steady-state ones); the empty asm keeps the loads above the wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  asm volatile("" ::: "memory");

  // whole groups of 4 steps: steps past d load zeros and add exact zeros
  int j = 0;
  do {
    load_sc(j + 1, sc_nxt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = 4 * j + u;
      const int p = u % PF;
      if constexpr (DMA) {
        // the loads issued after step s's x: the codes of step s+1, PF-2
        // steps of x and codes, and the next group's scale dwords where
        // those came later (u < PF-1)
        constexpr int base = NT + (PF - 2) * (SPT + NT);
        if (u < PF - 1) wait_vmcnt<base + NT>();
        else wait_vmcnt<base>();
        lds_dma_barrier();
        dma_x(s + PF - 1, (p + PF - 1) % PF);
      }
      // stage x of step s into slot p (last read at step s-PF, before the
      // previous barrier)
#pragma unroll
      for (int i = 0; i < (DMA ? 0 : SPT); ++i) {
        const bool live = tid + i * NTH < MAXC * 16;
        uint8_t *dst = live ? lds + p * SLOT + pcol[i] * kBRow + pel[i] * 2 : lds + dummy;
        const uint32_t pstep = live ? MAXC * kBRow : 16;
        if (XBF16) {
          *(u32x4 *)dst = xst[p][i][0];
        } else {
          uint32_t hi[8], mi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) split3_bf16(__uint_as_float(xst[p][i][e >> 2][e & 3]), hi[e], mi[e], lo[e]);
          u32x4 ph, pm, pl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
            pm[e] = mi[2 * e] | (mi[2 * e + 1] << 16);
            pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
          }
          *(u32x4 *)dst = ph;
          *(u32x4 *)(dst + pstep) = pm;
          *(u32x4 *)(dst + 2 * pstep) = pl;
        }
      }
      if constexpr (!DMA) lds_barrier();
      float sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((r + 16 * u) * 4, (int)sc_cur[t]);
        sc[t] = e8m0_to_f32((w >> (8 * q)) & 0xFFu);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x8 b[NCB][NP];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int pp = 0; pp < NP; ++pp)
            b[cb][pp] = DMA ? lds_b_fragment(lds, p * SLOTD + (16 * cb + r) * 256 + (((4 * q + jj) ^ r) << 4))
                            : lds_b_fragment(lds, p * SLOT + (pp * MAXC + 16 * cb + r) * kBRow + ((q << 5) + 8 * jj) * 2);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 a = fp4x8_to_bf16(ring[p][t][jj], sc[t]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) acc[t][cb] = mfma16x16x32(a, b[cb][pp], acc[t][cb]);
        }
      }
      issue(s + PF, p);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) sc_cur[t] = sc_nxt[t];
  } while (++j < ngroups);
  // DMA: no LDS write may land after the workgroup has ended
  if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // SwiGLU and the split of h into kHParts parts, as in ffn_gateup_kernel
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = 16 * cb + r;
    if (col < count) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = i0 + wv * 32 + 16 * t + 4 * q;
        if (row < f) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = acc[t][cb][i], uv = acc[t + 2][cb][i];
            split2_bf16((gv / (1.0f + expf(-gv))) * uv, hi[i], lo[i]);
          }
          uint16_t *hp = h_ws + (int64_t)(start + col) * kHParts * f + row;
          *(uint2 *)(hp) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
          *(uint2 *)(hp + f) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Workgroup = (group, DW*TPW*16 rows of d); each wave owns TPW row tiles and
// the whole f reduction.  B = the group's h in kHParts = 2 bf16 parts, two
// MFMA columns per slot: B row (global column) 2*j + p holds part p of slot j.
// Those are rows start*2 + 2*j + p of the workspace's h, one contiguous
// block for the group.  Columns come in blocks of 16, so a group of c slots
// takes ceil(2c/16) MFMAs per 32-element slice (one for up to 8 slots).
// Every column accumulates one (slot, part) over the whole reduction in a
// fixed order, independent of the column's position; the epilogue adds a
// slot's two part sums, hi + lo.  Lanes of columns past the group's read B
// row 0 (those columns are never used).
//
// SCR (ring mode, f % 128 == 0): the scales travel with the ring loads
// instead of being staged in LDS, as in the wide gate/up kernel: every 4
// steps lane (r, q) of a tile loads the dword of its row holding the 4
// block scales of step 4j + q, and at step 4j + u a bpermute from lane
// (r, u) hands lane (r, q) byte q (the same byte, the same 2^(b-127), as a
// staged scale).  The LDS it frees lets two wide workgroups share a CU.
//
// DMA (ring mode): B goes from the workspace straight into its ring slot
// with LDS DMA instead of through registers.  A slot holds the step's B rows
// at a 256-byte pitch, the 16-byte chunk c of row j at position c ^ (j % 16)
// (16 consecutive rows then spread a chunk column over all banks); lane l of
// a DMA instruction fills one chunk, choosing its source accordingly.  Slot
// (s-1) % PF is refilled with step s+PF-1 right after step s's barrier (the
// barrier that also tells every wave is done reading it), so B runs PF-1
// steps ahead and the codes PF steps.  Step s waits for its own DMA loads by
// count (wait_vmcnt; loads retire in issue order) before that barrier.
// Same bytes, same products, same order: bit-identical to register staging.
template <int TPW, int DW, int PF, int MAXC, bool SX4, bool BRES, int CS, bool SCR = false, bool DMA = false>
__global__ __launch_bounds__(DW * 64) void ffn_down_kernel(
    int d, int f, int n_slots, const uint8_t *__restrict__ experts, int64_t stride, GroupSrc src,
    const int32_t *__restrict__ perm, int n_dtiles, const uint16_t *__restrict__ h_ws, float *__restrict__ y) {
  constexpr int ROWS = DW / CS * TPW * 16;
  constexpr int NTH = DW * 64;
  constexpr int NC = kHParts * MAXC;  // B rows at most
  constexpr int NCB = (NC + 15) / 16;  // column blocks at most
  static_assert(DW % CS == 0 && NCB % CS == 0, "column split");
  constexpr int NCBW = NCB / CS;       // column blocks per wave
  constexpr int NPIECE = NC * 16;     // ring staging pieces per step (8 elements each)
  constexpr int SPT = BRES ? 0 : (NPIECE + NTH - 1) / NTH;
  constexpr int SPTA = SPT > 0 ? SPT : 1;
  constexpr int YC = down_yc(PF, MAXC, BRES, ROWS);  // epilogue columns per phase
  constexpr int SPP = YC / kHParts;                   // slots per phase
  constexpr int NPH = (MAXC + SPP - 1) / SPP;         // epilogue phases
  constexpr int YP = ROWS + 4;                        // epilogue column pitch (floats)
  static_assert(!SCR || (!BRES && 4 % PF == 0), "ring scales: ring mode, ring depth divides 4");
  static_assert(!DMA || (!BRES && PF >= 2 && NPIECE % NTH == 0), "LDS DMA: ring mode, whole 1 KB pieces per wave");
  constexpr uint32_t RP = DMA ? 256u : (uint32_t)kBRow;  // B row pitch in a ring slot
  constexpr uint32_t SLOTB = (uint32_t)NC * RP;          // bytes of one ring slot
  extern __shared__ __align__(16) uint8_t lds[];
  const int item = xcd_item(group_count(src) * n_dtiles);
  if (item < 0) return;
  const int g = item / n_dtiles;
  const int dt = item - g * n_dtiles;
  int expert, start, count;
  if (!load_group(src, g, expert, start, count, MAXC)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int cs = wv % CS, rgw = wv / CS;  // column part and row group of this wave
  const int nc = kHParts * count, ncb = (nc + 15) >> 4;
  const uint32_t plane = (uint32_t)((int64_t)f * d / 2 + (int64_t)f * d / 32);
  const uint32_t dn_c = 2 * plane, dn_s = dn_c + (uint32_t)((int64_t)d * f / 2);
  const rsrc_t wr = expert_rsrc(src, experts, stride, expert);
  const rsrc_t hr = make_rsrc(h_ws, (uint32_t)((int64_t)n_slots * kHParts * f * 2));
  const uint32_t hbase = (uint32_t)start * (uint32_t)(kHParts * f * 2);  // the group's first h row
  const int r0 = dt * ROWS;
  const uint32_t brow = bres_row_bytes(f);
  const uint32_t dummy = (uint32_t)down_dummy_off(f, PF, MAXC, BRES, ROWS, SCR);
  uint8_t *const bmem = lds + down_b_off(f, ROWS, SCR);  // B area (after the scale rows)
  int bsel[NCBW];  // B row read by this lane in each of its column blocks
#pragma unroll
  for (int cbl = 0; cbl < NCBW; ++cbl) {
    const int cb = cs * NCBW + cbl;
    bsel[cbl] = cb * 16 + r < nc ? cb * 16 + r : 0;
  }

  // ring staging pieces: piece i is B row i/16, elements 8*(i%16)..+8 of the step
  uint32_t pbase[SPTA];
  int prow[SPTA], pel[SPTA];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int piece = tid + i * NTH;
    prow[i] = piece >> 4;
    // DMA: the chunk stored at position piece % 16 of row prow
    pel[i] = DMA ? ((piece & 15) ^ (prow[i] & 15)) * 8 : (piece & 15) * 8;
    pbase[i] = (piece < NPIECE && prow[i] < nc) ? hbase + (uint32_t)prow[i] * (uint32_t)(f * 2) : kOOB;
  }
  uint32_t aoff[TPW];
  const uint8_t *srow[TPW];  // this lane's LDS scale row per tile
  uint32_t soff[TPW];        // SCR: this lane's scale dword of step q per tile
  const int nb = f >> 5;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int lrow = (rgw * TPW + t) * 16 + r;
    const int row = r0 + lrow;
    aoff[t] = sel_off(row < d, dn_c + code_off(src, row, r, q, f));
    srow[t] = lds + lrow * sc_pitch(f);
    soff[t] = sel_off(row < d, dn_s + (uint32_t)row * (uint32_t)nb + 4u * q);
  }
  f32x4 acc[TPW][NCBW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int cbl = 0; cbl < NCBW; ++cbl) acc[t][cbl] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (f + 127) >> 7;
  const int smax = (f - (q << 5) + 127) >> 7;
  u32x4 ring[PF][TPW];
  u32x4 hst[PF][DMA ? 1 : SPTA];
  const uint32_t cstep = code_step(src);
  auto issue = [&](int s, int p) {
    const uint32_t ka = s < smax ? (uint32_t)s * cstep : kDead;
#pragma unroll
    for (int t = 0; t < TPW; ++t) ring[p][t] = MAXC <= kGroupCols ? buf_load16_stream(wr, aoff[t] + ka) : buf_load16(wr, aoff[t] + ka);
    if constexpr (!DMA) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int k = (s << 7) + pel[i];
        hst[p][i] = buf_load16(hr, pbase[i] + (k < f ? (uint32_t)(k * 2) : kDead));
      }
    }
  };
  // DMA: B of step s into ring slot p, one 1 KB piece per wave instruction
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  auto dma_b = [&](int s, int p) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int k = (s << 7) + pel[i];
      buf_load16_lds(hr, pbase[i] + (k < f ? (uint32_t)(k * 2) : kDead), bmem + p * SLOTB + (uint32_t)(i * NTH + wvu * 64) * 16u);
    }
  };
  // SCR: the scale dwords of step group j (4 steps); a padding step's dword
  // would lie past the row's f/32 scale bytes, so such lanes read past the
  // resource (zero bytes) instead (see the wide gate/up kernel)
  const int ngroups4 = (nsteps + 3) >> 2;
  uint32_t sc_cur[TPW], sc_nxt[TPW];
  auto load_sc = [&](int j, uint32_t (&scv)[TPW]) {
    const uint32_t js = (j < ngroups4 && 4 * j + q < nsteps) ? 16u * (uint32_t)j : kDead;
#pragma unroll
    for (int t = 0; t < TPW; ++t) scv[t] = buf_load4(wr, soff[t] + js);
  };
  // scale staging loads, then the ring prefill, one wait (see the gate/up kernel)
  const int rv = d - r0 < ROWS ? d - r0 : ROWS;
  ScaleStage<SX4, !BRES> ss;
  if constexpr (SCR) load_sc(0, sc_cur);
  else ss.begin(wr, dn_s, r0, rv, ROWS, f, tid, NTH);
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, p);
  if constexpr (DMA) {
#pragma unroll
    for (int p = 0; p < PF - 1; ++p) dma_b(p, p);
  }
  asm volatile("" ::: "memory");
  if constexpr (!BRES) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  asm volatile("" ::: "memory");
  if constexpr (!SCR) ss.end(wr, dn_s, r0, rv, ROWS, f, lds, dummy, lds, tid, NTH);
  if constexpr (BRES) {
    // the group's nc h rows for the whole f, all loads of a round issued first
    constexpr int CH = 8;
    const int per_row = f / 8;
    const int npieces = nc * per_row;
    for (int base = 0; base < npieces; base += CH * NTH) {
      u32x4 v[CH];
      int pr[CH], pe[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int piece = base + c * NTH + tid;
        pr[c] = piece / per_row;
        pe[c] = (piece - pr[c] * per_row) * 8;
        v[c] = buf_load16(hr, piece < npieces ? hbase + (uint32_t)(pr[c] * f + pe[c]) * 2u : kOOB);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c)
        *(u32x4 *)(base + c * NTH + tid < npieces ? bmem + pr[c] * brow + pe[c] * 2 : lds + dummy) = v[c];
    }
    for (int idx = tid; idx < nc * (kBresTail / 16); idx += NTH) {
      const int row = idx / (kBresTail / 16), c = idx - row * (kBresTail / 16);
      *(u32x4 *)(bmem + row * brow + f * 2 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
    lds_barrier();
  }

  // one step: stage B of step s into ring slot p, then its MFMAs, then the
  // refill of slot p.  The scales are the ring's (SCR: sc_ring) or read from
  // LDS after the step's barrier, which on the first step also publishes the
  // staged scale rows of every wave.
  // DMA: loads issued after step s's B, by position u of s in its group of 4
  // steps (ring scales): the codes of step s+1, then PF-2 steps of B and
  // codes, plus the scale dwords of the next group where those were issued
  // after step s's B (u < PF-1)
  auto wait_b = [&](int u) {
    constexpr int base = TPW + (PF - 2) * (SPT + TPW);
    if (SCR && u < PF - 1) wait_vmcnt<base + TPW>();
    else wait_vmcnt<base>();
  };
  auto step = [&](int s, int p, const float (&sc_ring)[TPW], int u) {
      if constexpr (DMA) {
        wait_b(u);
        lds_dma_barrier();
        dma_b(s + PF - 1, (p + PF - 1) % PF);
      } else {
#pragma unroll
        for (int i = 0; i < SPT; ++i)
          *(u32x4 *)(tid + i * NTH < NPIECE ? bmem + (p * NC + prow[i]) * kBRow + pel[i] * 2 : lds + dummy) = hst[p][i];
        if constexpr (!BRES) lds_barrier();
      }
      float sc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[t] = SCR ? sc_ring[t] : lds_scale(srow[t], s, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 a[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) a[t] = fp4x8_to_bf16(ring[p][t][j], sc[t]);
#pragma unroll
        for (int cbl = 0; cbl < NCBW; ++cbl) {
          // narrow groups skip their empty column blocks; wide groups are
          // nearly full and run straight-line code (the extra columns read
          // B row 0 and are never stored)
          if (MAXC > 16 || cs * NCBW + cbl < ncb) {
            bf16x8 b;
            if constexpr (BRES)
              b = lds_b_fragment(bmem, bsel[cbl] * brow + (s < smax ? ((s << 7) + (q << 5) + 8 * j) * 2 : f * 2 + 16 * j));
            else if constexpr (DMA)
              b = lds_b_fragment(bmem, p * SLOTB + bsel[cbl] * RP + (((4 * q + j) ^ (bsel[cbl] & 15)) << 4));
            else
              b = lds_b_fragment(bmem, (p * NC + bsel[cbl]) * kBRow + ((q << 5) + 8 * j) * 2);
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t][cbl] = mfma16x16x32(a[t], b, acc[t][cbl]);
          }
        }
      }
      issue(s + PF, p);
      // keep the refill here: the scheduler would otherwise sink it past the
      // next steps' waits and drain the ring once per unrolled window
      __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (SCR) {
    // whole groups of 4 steps: steps past f load zeros and add exact zeros
    int j = 0;
    do {
      load_sc(j + 1, sc_nxt);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float sc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((r + 16 * u) * 4, (int)sc_cur[t]);
          sc[t] = e8m0_to_f32((w >> (8 * q)) & 0xFFu);
        }
        step(4 * j + u, u % PF, sc, u);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc_cur[t] = sc_nxt[t];
    } while (++j < ngroups4);
  } else {
    const int nsteps_pad = (nsteps + PF - 1) / PF * PF;  // see the gate/up kernel
    const float none[TPW] = {};
    for (int s0 = 0; s0 < nsteps_pad; s0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) step(s0 + p, p, none, PF);
    }
  }

  // every (row, column) sum goes through LDS (in the B area: all waves are
  // past their last B read at the first barrier), SPP slots (YC columns) per
  // phase, column-major: a lane stores the 4 rows it holds of its column as
  // one float4, and a thread reads 4 consecutive rows of a slot's two part
  // columns as two float4 (a pitch of ROWS + 4 floats puts both on distinct
  // banks across 16 lanes); each slot's part sums are added in a fixed
  // order (hi + lo) and its rows written as float4
  // DMA: every ring load (the padded steps' too) has landed before the B
  // area is reused
  if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  float *ys = (float *)(lds + down_y_off(f, PF, MAXC, BRES, ROWS, SCR));
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) {
    lds_barrier();
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int cbl = 0; cbl < NCBW; ++cbl) {
        const int col = (cs * NCBW + cbl) * 16 + r;
        if (col >= YC * ph && col < YC * (ph + 1) && col < nc)
          *(f32x4 *)(ys + (col - YC * ph) * YP + (rgw * TPW + t) * 16 + 4 * q) = acc[t][cbl];
      }
    lds_barrier();
    const int j0 = SPP * ph, nj = count - j0 < SPP ? count - j0 : SPP;
    for (int idx = tid; idx < nj * (ROWS / 4); idx += NTH) {
      const int jl = idx / (ROWS / 4), lrow = (idx - jl * (ROWS / 4)) * 4;
      const int row = r0 + lrow;
      const int t_slot = perm[start + j0 + jl];
      if (row < d && t_slot >= 0 && t_slot < n_slots) {
        const f32x4 hi = *(const f32x4 *)(ys + (kHParts * jl) * YP + lrow);
        const f32x4 lo = *(const f32x4 *)(ys + (kHParts * jl + 1) * YP + lrow);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = hi[i] + lo[i];
        *(f32x4 *)(y + (int64_t)t_slot * d + row) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ host side
static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Group list capacities with many rows: narrow groups (at most ceil(T/16) +
// one per expert when every group is narrow), 32-wide (at most one per
// expert, at least 17 slots each) and 64-wide (at least 33 slots each).
static void group_caps(int64_t M, int k, int S, int n_experts, int64_t cap[kGroupClasses]) {
  const int64_t T = M * (k + S);
  cap[0] = (T + kGroupCols - 1) / kGroupCols + n_experts;
  cap[1] = std::min<int64_t>(n_experts, T / 17);
  cap[2] = T / 33;
}

int64_t ffn_max_groups(int64_t M, int k, int S, int n_experts) {
  const int64_t T = M * (k + S);
  if (M <= kGroupCols) return n_experts < T ? n_experts : T;
  int64_t cap[kGroupClasses];
  group_caps(M, k, S, n_experts, cap);
  return cap[0] + cap[1] + cap[2];
}

size_t ffn_workspace_bytes(int64_t M, int k, int S, int d, int f, int n_experts) {
  const int64_t T = M * (k + S);
  size_t b = align_up((size_t)T * kHParts * f * sizeof(uint16_t), 256);
  if (M > kGroupCols) {
    int64_t cap[kGroupClasses];
    group_caps(M, k, S, n_experts, cap);
    for (int c = 0; c < kGroupClasses; ++c) b += align_up((size_t)cap[c] * sizeof(int4), 256);
  }
  b += 256;  // group counts
  (void)d;
  return b;
}

// gfx950 gives a workgroup up to 160 KB of LDS; kernels opt in past 64 KB.
constexpr int kMaxLds = 160 * 1024;
static bool allow_lds(const void *kernel, int bytes = kMaxLds) {
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess) return true;
  (void)hipGetLastError();  // leave no error behind for the next launch check
  return false;
}
// Route-mode kernels hold a few bytes of static LDS besides the dynamic area.
constexpr int kRouteMaxLds = kMaxLds - 1024;

// Every buffer resource must stay below 2^30 bytes (see kOOB / kDead).
bool ffn_shape_ok(int64_t M, int k, int S, int d, int f, int64_t stride) {
  const int64_t T = M * (k + S);
  const int64_t lim = (int64_t)kDead;
  (void)d;
  (void)f;
  return stride < lim &&
         M * (int64_t)d * 4 < lim && T * kHParts * f * 2 < lim;
}

template <int XBF16, int TPW, int GW, int PF, int MAXC, bool SX4, bool BRES, bool PAIR, bool ROUTE = false>
static int launch_gateup(const void *x, int d, int f, int kps, int T, const uint8_t *experts, int64_t stride,
                         const GroupSrc &src, const int32_t *perm, int64_t maxg, uint16_t *h_ws, hipStream_t stream,
                         const RouteArgs &ra = RouteArgs{}) {
  constexpr int ROWS = (PAIR ? GW : GW / 2) * TPW * 16;
  const int n_ftiles = (f + ROWS - 1) / ROWS;
  if (maxg <= 0) return 0;
  size_t smem = gateup_lds_bytes(d, PF, XBF16 ? 1 : 3, MAXC, BRES, ROWS);
  if (ROUTE) smem = std::max(smem, topk_wave_lds(16));  // the ranking lists alias the start of LDS
  if (smem > (size_t)(ROUTE ? kRouteMaxLds : kMaxLds)) return -3;
  static const bool lds_ok =
      allow_lds(reinterpret_cast<const void *>(&ffn_gateup_kernel<XBF16, TPW, GW, PF, MAXC, SX4, BRES, PAIR, ROUTE>),
                ROUTE ? kRouteMaxLds : kMaxLds);
  if (!lds_ok) return -3;
  hipLaunchKernelGGL((ffn_gateup_kernel<XBF16, TPW, GW, PF, MAXC, SX4, BRES, PAIR, ROUTE>), dim3((unsigned)align_up((size_t)(maxg * n_ftiles), kXcds)), dim3(GW * 64),
                     smem, stream, x, d, f, kps, T, experts, stride, src, perm, n_ftiles, h_ws, ra);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int XBF16, int GW, int PF, int NCB, bool DMA = false>
static int launch_gateup_wide(const void *x, int d, int f, int kps, int T, const uint8_t *experts, int64_t stride,
                              const GroupSrc &src, const int32_t *perm, int64_t maxg, uint16_t *h_ws,
                              hipStream_t stream) {
  constexpr int ROWS = GW * 32;
  const int n_ftiles = (f + ROWS - 1) / ROWS;
  if (maxg <= 0) return 0;
  // LDS DMA: every ring slot filled by a real step before a padded step reads it
  if (DMA && d < 128 * PF) return -3;
  const size_t smem = (size_t)PF * (XBF16 ? 1 : 3) * 16 * NCB * kBRow + 48;
  if (smem > (size_t)kMaxLds) return -3;
  static const bool lds_ok = allow_lds(reinterpret_cast<const void *>(&ffn_gateup_wide_kernel<XBF16, GW, PF, NCB, DMA>));
  if (!lds_ok) return -3;
  hipLaunchKernelGGL((ffn_gateup_wide_kernel<XBF16, GW, PF, NCB, DMA>), dim3((unsigned)align_up((size_t)(maxg * n_ftiles), kXcds)), dim3(GW * 64),
                     smem, stream, x, d, f, kps, T, experts, stride, src, perm, n_ftiles, h_ws);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int TPW, int DW, int PF, int MAXC, bool SX4, bool BRES, int CS, bool SCR = false, bool DMA = false>
static int launch_down(int d, int f, int T, const uint8_t *experts, int64_t stride, const GroupSrc &src,
                       const int32_t *perm, int64_t maxg, const uint16_t *h_ws, float *y, hipStream_t stream) {
  constexpr int ROWS = DW / CS * TPW * 16;
  const int n_dtiles = (d + ROWS - 1) / ROWS;
  if (maxg <= 0) return 0;
  if (SCR && f % 128) return -3;
  // LDS DMA: whole steps only, and every ring slot filled by a real step
  // before a padded step reads it
  if (DMA && (f % 128 || f < 128 * PF)) return -3;
  const size_t smem = down_lds_bytes(f, PF, MAXC, BRES, ROWS, SCR);
  if (smem > (size_t)kMaxLds) return -3;
  static const bool lds_ok =
      allow_lds(reinterpret_cast<const void *>(&ffn_down_kernel<TPW, DW, PF, MAXC, SX4, BRES, CS, SCR, DMA>));
  if (!lds_ok) return -3;
  hipLaunchKernelGGL((ffn_down_kernel<TPW, DW, PF, MAXC, SX4, BRES, CS, SCR, DMA>), dim3((unsigned)align_up((size_t)(maxg * n_dtiles), kXcds)), dim3(DW * 64), smem,
                     stream, d, f, T, experts, stride, src, perm, n_dtiles, h_ws, y);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The one-row gate/up shapes that route mode runs in (see ffn_launch).
static bool gateup_one_row_bres(int x_bf16, int d) {
  const size_t half = (size_t)kMaxLds / 2;
  return x_bf16 ? gateup_lds_bytes(d, 4, 1, 1, true, 64) <= half : gateup_lds_bytes(d, 4, 3, 4, true, 32) <= half;
}

bool ffn_route_fusable(int64_t M, int x_bf16, int d, int E, int k, int S) {
  return M == 1 && E <= 16 * 64 && k + S <= 64 && E + S + 1 <= 64 * 64 && gateup_one_row_bres(x_bf16, d);
}

int ffn_launch(const void *x, int x_bf16, int64_t M, int k, const uint8_t *experts, int64_t stride, int d, int f,
               int n_routed, int n_shared, const int32_t *offsets, const int32_t *perm, const int32_t *active,
               const int32_t *n_active, float *y, void *workspace, int stages, const int32_t *slot_map,
               int n_records, int64_t max_active, int tiled, hipStream_t stream, const RouteArgs *route) {
  if (route && (!ffn_route_fusable(M, x_bf16, d, n_routed, k, n_shared) || !(stages & kStageGateUp) || slot_map))
    return -3;
  const int S = n_shared;
  const int kps = k + S;
  const int64_t T = M * kps;
  const int n_experts = n_routed + n_shared;
  uint8_t *ws = (uint8_t *)workspace;
  uint16_t *h_ws = (uint16_t *)ws;
  size_t off = align_up((size_t)T * kHParts * f * sizeof(uint16_t), 256);
  const bool many = M > kGroupCols;
  // with many rows: groups of up to 64 slots where the wide gate/up kernel
  // applies (dword-aligned scale rows)
  const bool wide = many && d % 128 == 0;
  int64_t cap[kGroupClasses] = {ffn_max_groups(M, k, S, n_experts), 0, 0};
  // with few rows a group is an active expert: a known bound on them sizes the grids
  if (max_active > 0 && M <= kGroupCols) cap[0] = std::min<int64_t>(cap[0], max_active);
  int4 *glist[kGroupClasses] = {nullptr, nullptr, nullptr};
  if (many) {
    group_caps(M, k, S, n_experts, cap);
    for (int c = 0; c < kGroupClasses; ++c) {
      glist[c] = (int4 *)(ws + off);
      off += align_up((size_t)cap[c] * sizeof(int4), 256);
    }
    if (!wide) cap[1] = cap[2] = 0;
    // grids (not list capacities): with wide groups every active expert has
    // at most one narrow group (itself, or the remainder of its 64s), so the
    // narrow kernels need not launch ceil(T/16) + E groups' workgroups, most
    // of which would find no group
    if (wide) cap[0] = std::min<int64_t>(cap[0], std::min<int64_t>(n_experts, T));
  }
  int32_t *n_groups = (int32_t *)(ws + off);

  GroupSrc src[kGroupClasses];
  for (int c = 0; c < kGroupClasses; ++c)
    src[c] = GroupSrc{offsets, active, n_active, nullptr, nullptr, slot_map, n_records, tiled};
  if (many) {
    // the group plan lives in the workspace and serves both stages
    if (stages & kStageGateUp) {
      hipLaunchKernelGGL(plan_groups_kernel, dim3(1), dim3(1024), 0, stream, offsets, active, n_active, glist[0],
                         glist[1], glist[2], n_groups, wide ? 1 : 0);
      if (hipGetLastError() != hipSuccess) return -3;
    }
    for (int c = 0; c < kGroupClasses; ++c) {
      src[c].groups = glist[c];
      src[c].n_groups = n_groups + c;
    }
  }
  // Launch shapes only change how many rows a wave/workgroup owns and how
  // many B columns are staged (a group never has more slots than its kernel's
  // column limit), never the order of any reduction: every choice gives
  // bit-identical results.
  const bool gsx4 = (d / 32) % 16 == 0, dsx4 = (f / 32) % 16 == 0;
  const int T_ = (int)T;
#define MOE_GU(XB, T, G, P, C, R, PR)                                                                          \
  (gsx4 ? launch_gateup<XB, T, G, P, C, true, R, PR>(x, d, f, kps, T_, experts, stride, src[0], perm, cap[0], h_ws, stream) \
        : launch_gateup<XB, T, G, P, C, false, R, PR>(x, d, f, kps, T_, experts, stride, src[0], perm, cap[0], h_ws, stream))
#define MOE_GUR(XB, T, G, P, C)                                                                                  \
  (gsx4 ? launch_gateup<XB, T, G, P, C, true, true, true, true>(x, d, f, kps, T_, experts, stride, src[0], perm,   \
                                                                 cap[0], h_ws, stream, *route)                    \
        : launch_gateup<XB, T, G, P, C, false, true, true, true>(x, d, f, kps, T_, experts, stride, src[0], perm,  \
                                                                  cap[0], h_ws, stream, *route))
#define MOE_GUW(XB, G, P, NCB, CL) \
  launch_gateup_wide<XB, G, P, NCB>(x, d, f, kps, T_, experts, stride, src[CL], perm, cap[CL], h_ws, stream)
  // bf16 x through LDS DMA (d >= 512 fills the 4-step ring)
#define MOE_GUWD(G, P, NCB, CL) \
  launch_gateup_wide<1, G, P, NCB, true>(x, d, f, kps, T_, experts, stride, src[CL], perm, cap[CL], h_ws, stream)
#define MOE_DNR(T, D, P, C, CL, CS)                                                                                    \
  (dsx4 ? launch_down<T, D, P, C, true, false, CS, true>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, y,     \
                                                          stream)                                                       \
        : launch_down<T, D, P, C, false, false, CS, true>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, y,    \
                                                           stream))
#define MOE_DN(T, D, P, C, R, CL, CS)                                                                                   \
  (dsx4 ? launch_down<T, D, P, C, true, R, CS>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, y, stream) \
        : launch_down<T, D, P, C, false, R, CS>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, y, stream))
  // ring mode with B through LDS DMA: scales through the ring (SCR) or staged
#define MOE_DND(T, D, P, C, CL, CS, SCRV)                                                                               \
  (dsx4 ? launch_down<T, D, P, C, true, false, CS, SCRV, true>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, \
                                                                y, stream)                                              \
        : launch_down<T, D, P, C, false, false, CS, SCRV, true>(d, f, T_, experts, stride, src[CL], perm, cap[CL], h_ws, \
                                                                 y, stream))
  // few rows: each group's B operand (x or h) stays resident in LDS for the
  // whole reduction; more rows: B is staged step by step through a ring.
  // Launch shapes (measured at the Kimi shape on tile-ordered records):
  // gate/up 4 waves each with the W_gate and W_up tiles of 16 rows (64 rows
  // of f) and a 4-step ring at 1-2 rows, 4 waves (half W_gate, half W_up) at
  // 5-8 rows, 4 waves each with both tiles again beyond (4-step rings), and
  // the wide kernel (8 waves x 32 rows) for the 32- and 64-slot groups;
  // down 4 waves x 2 tiles (128 rows of d) at 1-4 rows, 4 waves x 2 tiles
  // and a 2-step ring up to 16 rows (LDS DMA), 8 waves x 4 tiles (512 rows)
  // with a 2-step ring for the narrow groups of more rows, and 8 waves x 2
  // tiles for the wide groups.  A resident B is used only where the LDS it
  // takes still lets two or more workgroups share a CU.
  int rc = 0;
  if (stages & kStageGateUp) {
    const int np = x_bf16 ? 1 : 3;
    const size_t half = (size_t)kMaxLds / 2;
    if (route) {
      // one row, groups from the logits (ffn_route_fusable checked the shape)
      cap[0] = k + S;
      rc = x_bf16 ? MOE_GUR(1, 1, 4, 4, 1) : MOE_GUR(0, 1, 2, 4, 4);
    } else if (x_bf16) {
      if (M == 1 && gateup_lds_bytes(d, 4, np, 1, true, 64) <= half) rc = MOE_GU(1, 1, 4, 4, 1, true, true);
      else if (M == 2 && gateup_lds_bytes(d, 4, np, 2, true, 64) <= half) rc = MOE_GU(1, 1, 4, 4, 2, true, true);
      else if (M >= 5 && M <= 8) rc = MOE_GU(1, 1, 4, 4, 16, false, false);
      // more rows: 4 waves each with the W_gate and W_up tiles of the same
      // 16 rows (measured against 8 waves split into W_gate and W_up: 16-row
      // block 181.6 -> 178-180 us, 1,533-row prefill 4.64 -> 4.59-4.61 ms)
      else rc = MOE_GU(1, 1, 4, 4, 16, false, true);
      // wide groups: x by LDS DMA where d fills the ring (1,533-row prefill,
      // wide gate/up 2.44 -> 2.42 ms, bit-identical)
      const bool gdma = d >= 512;
      if (!rc && wide) rc = gdma ? MOE_GUWD(8, 4, 2, 1) : MOE_GUW(1, 8, 4, 2, 1);
      if (!rc && wide) rc = gdma ? MOE_GUWD(8, 4, 4, 2) : MOE_GUW(1, 8, 4, 4, 2);
    } else {
      if (M <= 4 && gateup_lds_bytes(d, 4, np, 4, true, 32) <= half) rc = MOE_GU(0, 1, 2, 4, 4, true, true);
      else rc = MOE_GU(0, 1, 8, 4, 16, false, false);
      if (!rc && wide) rc = MOE_GUW(0, 8, 2, 2, 1);
      if (!rc && wide) rc = MOE_GUW(0, 8, 2, 4, 2);
    }
    if (rc) return rc;
  }
  if (stages & kStageDown) {
    const size_t half = (size_t)kMaxLds / 2;
    // ring mode: B by LDS DMA where f is whole steps of 128 and fills the
    // ring (f >= 512 covers every ring below); measured on MI355X at the
    // Kimi shape: 1,533-row prefill 4.86-4.88 -> 4.78-4.83 ms, blocks of 8
    // and 16 rows 0-4 us faster, bit-identical everywhere; up to 16 rows 4
    // waves x 2 tiles (16-row block 183-185 -> 182 us in a 5-shape sweep)
    const bool dma = f % 128 == 0 && f >= 512;
    // resident B, 4 waves x 2 tiles (128 rows of d): 1 row with a 2-step
    // ring, 2-4 rows with a 4-step ring (measured against 8 waves: 1 row
    // 69.7 -> 69.05 us, 2 rows 94 -> 90 us; a sweep of 11 shapes)
    if (M == 1 && down_lds_bytes(f, 2, 1, true, 128) <= half) rc = MOE_DN(2, 4, 2, 1, true, 0, 1);
    else if (M <= 4 && down_lds_bytes(f, 4, 4, true, 128) <= half) rc = MOE_DN(2, 4, 4, 4, true, 0, 1);
    else if (M <= kGroupCols) rc = dma ? MOE_DND(2, 4, 2, 16, 0, 1, false) : MOE_DN(2, 8, 4, 16, false, 0, 1);
    // more rows (the prefill's narrow groups): scales through the ring where
    // f % 128 == 0 (measured 4.90 -> 4.84 ms at 1,533 rows; at 16 rows the
    // staged scales are faster, 191.5 against 197.6 us)
    else rc = dma ? MOE_DND(4, 8, 2, 16, 0, 1, true) : f % 128 == 0 ? MOE_DNR(4, 8, 2, 16, 0, 1) : MOE_DN(4, 8, 2, 16, false, 0, 1);
    // the wide groups (MFMA-bound): scales through the ring where f % 128 == 0
    // (two workgroups a CU), else staged; with LDS DMA 2 tiles per wave
    // (128 rows of d for 64 slots, 256 for 32): a sweep at 1,533 rows gave
    // 4.64-4.66 -> 4.51-4.53 ms against the 4-tile shapes
    const bool scr = f % 128 == 0;
    if (!rc && wide) rc = dma ? MOE_DND(2, 8, 2, 32, 1, 1, true) : scr ? MOE_DNR(4, 8, 4, 32, 1, 2) : MOE_DN(4, 8, 4, 32, false, 1, 2);
    if (!rc && wide) rc = dma ? MOE_DND(2, 8, 2, 64, 2, 2, true) : scr ? MOE_DNR(4, 8, 2, 64, 2, 2) : MOE_DN(4, 8, 2, 64, false, 2, 2);
  }
#undef MOE_GU
#undef MOE_GUR
#undef MOE_GUW
#undef MOE_GUWD
#undef MOE_DN
#undef MOE_DND
#undef MOE_DNR
  return rc;
}

}  // namespace moe
