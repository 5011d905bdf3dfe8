// Top-k of one row of router logits in one wave, with the renormalised
// softmax weights of the selected experts ("Run Kimi 3.1 locally on one
// GPU", section "Read the experts the router needs": k = 16 routed experts
// out of E = 896 per token in the Kimi layer).  Shared by the top-k kernel and the fused
// top-k + bucket kernel, so both give the same bits.
//
// The row's logits sit in registers (NPL per lane).  Each entry becomes a
// 64-bit key: high word = the logit's bits mapped to an unsigned order (NaN
// as -inf, -0 as +0), low word = ~index, so a larger key is a larger logit or,
// on equal logits, a lower index.  k rounds take the wave maximum (a total
// order: every lane agrees) and retire it.
#pragma once
#include "common.h"

namespace moe {

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

// Lane j < k holds the logit and id of rank j: the weights
// exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), the normaliser summed in rank order.
__device__ __forceinline__ void topk_weights(float my_l, int32_t my_id, int lane, int k, int32_t &id_out,
                                             float &w_out) {
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float ej = (lane < k) ? expf(my_l - l0) : 0.f;
  float z = 0.f;
  for (int i = 0; i < k; ++i) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ej), i));
  id_out = my_id;
  w_out = ej / z;
}

// Keys per lane list: NPL rounded up to a power of two.
__host__ __device__ constexpr int topk_list_len(int npl) {
  return npl <= 1 ? 1 : npl <= 2 ? 2 : npl <= 4 ? 4 : npl <= 8 ? 8 : npl <= 16 ? 16 : npl <= 32 ? 32 : 64;
}
// LDS of one ranking wave: (P + 1) x 64 keys.
__host__ __device__ constexpr size_t topk_wave_lds(int npl) { return (size_t)(topk_list_len(npl) + 1) * 64 * 8; }

// Ranks row `row` (E logits) in the calling wave.  Lane l sorts the keys of
// entries l, l+64, ... largest first (P = topk_list_len(NPL), padded with key
// 0, which is below every real key) and parks the sorted list in `lists`
// (this wave's [P + 1][64] keys), keeping its first two keys in registers.
// Each round takes the largest head over the wave; the owning lane (keys are
// distinct: the index is part of the key) moves on to its next key.  Lane j < k
// gets the expert of rank j and its weight exp(l_j - l_0) / sum_{i<k}
// exp(l_i - l_0), the normaliser summed in rank order.
template <int NPL>
__device__ __forceinline__ void topk_row(const float *__restrict__ row, int E, int k, uint64_t (*lists)[64], int lane,
                                         int32_t &id_out, float &w_out) {
  constexpr int P = topk_list_len(NPL);
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
#pragma unroll
  for (int i = 2; i < P; ++i) lists[i][lane] = key[i];
  lists[P][lane] = 0ull;  // past the end of every list
  // the head and the key after it stay in registers: a lane that wins a
  // round promotes its next key and starts the LDS read of the one after,
  // which is needed a round later at the earliest
  uint64_t head = key[0], nxt = P > 1 ? key[P > 1 ? 1 : 0] : 0ull;
  int pos = P > 1 ? 1 : P;  // index of nxt in this lane's list
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
      head = nxt;
      pos = pos < P ? pos + 1 : P;
      nxt = lists[pos][lane];
    }
    if (lane == j) {
      my_l = from_order_bits(hmax);
      my_id = (int32_t)~lmax;
    }
  }
  topk_weights(my_l, my_id, lane, k, id_out, w_out);
}

// The same top-k by a threshold: every key is at most its lane's maximum, so
// the k-th largest key is at least the k-th largest of the 64 lane maxima,
// and in particular its top 16 bits are at least t, the k-th largest top 16
// bits among the lane maxima (found 4 bits at a time: 15 wave ballots per
// step, one count each).  The keys whose top 16 bits are at least t are
// gathered in LDS; when there are at most 64 of them (the usual case: logits
// that share the threshold's sign, exponent and 7 mantissa bits are few)
// each is ranked by counting the larger ones, else the list-based rounds
// above run.  Keys are distinct, so the k largest and their order are the
// same either way, and the weights are computed by the same code from the
// same values (skipped when `need_w` is false: w_out is then 0).  `lists`: at
// least topk_wave_lds(NPL) bytes of this wave's LDS.
template <int NPL>
__device__ __forceinline__ void topk_row_fast(const float *__restrict__ row, int E, int k, uint64_t (*lists)[64],
                                              int lane, int32_t &id_out, float &w_out, bool need_w = true) {
  static_assert(NPL >= 2, "the candidate, ranked and spill keys need 144 keys of LDS");
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
  uint64_t key[NPL];
  uint64_t m = 0ull;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (((uint64_t)order_bits(v[i]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
    m = max_u64(m, key[i]);
  }
  // t: the largest 16-bit value with at least k lane maxima at or above it
  const uint32_t mh = (uint32_t)(m >> 48);
  uint32_t t = 0;
#pragma unroll
  for (int sh = 12; sh >= 0; sh -= 4) {
    uint32_t best = 0;
#pragma unroll
    for (uint32_t d = 1; d < 16; ++d)
      best = __popcll(__ballot(mh >= (t | (d << sh)))) >= (uint32_t)k ? d : best;
    t |= best << sh;
  }
  // gather the keys at or above t (key 0 marks an entry past E); slots past
  // the count read as key 0, which is below every real key; entries that do
  // not qualify, or past 64, go to a spill slot that nothing reads
  uint64_t *cand = &lists[0][0];  // [64 + 8] keys, then the k ranked keys, then 8 spill slots
  uint64_t *ranked = cand + 72;
  uint64_t *spill = cand + 136;
  cand[lane] = 0ull;
  if (lane < 8) cand[64 + lane] = 0ull;
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool c = key[i] != 0ull && (uint32_t)(key[i] >> 48) >= t;
    const uint64_t msk = __ballot(c);
    const int slot = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
    *(c && slot < 64 ? cand + slot : spill + (lane & 7)) = key[i];
    n += (int)__popcll(msk);
  }
  if (n > 64) {  // uniform: too many near the threshold
    topk_row<NPL>(row, E, k, lists, lane, id_out, w_out);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // rank of candidate `lane`: the number of larger candidates
  const uint64_t mine = lane < n ? cand[lane] : 0ull;
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += cand[j0 + u] > mine;
  }
  *(lane < n && rank < k ? ranked + rank : spill + (lane & 7)) = mine;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  float my_l = 0.f;
  int32_t my_id = 0;
  if (lane < k) {
    const uint64_t kj = ranked[lane];
    my_l = from_order_bits((uint32_t)(kj >> 32));
    my_id = (int32_t)~(uint32_t)kj;
  }
  if (need_w) {
    topk_weights(my_l, my_id, lane, k, id_out, w_out);
  } else {
    id_out = my_id;
    w_out = 0.f;
  }
}

// Bucketing of one row in one wave, from its top-k ids (lane j < k holds
// the expert of rank j, every id in [0, E)).  The row's k routed and S shared
// experts are distinct, so slot t's position in bucket order is the number
// of the row's experts below its own, and offsets[e] is the number of them
// below e.  Lane l writes offsets[l*C .. l*C+C) (C = ceil((E+S+1)/64)) from
// that count at l*C and a mask of the experts inside its range.  Needs
// k + S <= 64 and E + S + 1 <= 4096; the results equal the general
// counting sort's.
__device__ __forceinline__ void bucket_one_row(int32_t id, int lane, int E, int k, int S, int32_t *offsets,
                                               int32_t *perm, int32_t *active, int32_t *n_active,
                                               int32_t *dev_error) {
  const int kps = k + S, NE = E + S;
  const int e_t = lane < k ? id : (lane < kps ? E + (lane - k) : 0x7FFFFFFF);
  const int C = (NE + 1 + 63) >> 6, e0 = lane * C;
  int rank = 0, below = 0;
  uint64_t inside = 0ull;
  for (int u = 0; u < kps; ++u) {
    const int eu = __builtin_amdgcn_readlane(e_t, u);
    rank += eu < e_t;
    below += eu < e0;
    const int rel = eu - e0;
    if (rel >= 0 && rel < C) inside |= 1ull << rel;
  }
  if (lane < kps) {
    perm[rank] = lane;
    active[rank] = e_t;
  }
  for (int i = 0; i < C; ++i)
    if (e0 + i <= NE) offsets[e0 + i] = below + __popcll(inside & ((1ull << i) - 1ull));
  if (lane == 0) {
    *n_active = kps;
    *dev_error = 0;
  }
}

// The ranking every kernel uses: the threshold form where a lane holds two or
// more logits, the list rounds otherwise (their LDS is too small for the
// threshold form's 136 keys).  Both give the same ids and weights.
template <int NPL>
__device__ __forceinline__ void topk_row_any(const float *__restrict__ row, int E, int k, uint64_t (*lists)[64],
                                             int lane, int32_t &id_out, float &w_out, bool need_w = true) {
  if constexpr (NPL >= 2)
    topk_row_fast<NPL>(row, E, k, lists, lane, id_out, w_out, need_w);
  else
    topk_row<NPL>(row, E, k, lists, lane, id_out, w_out);
}

}  // namespace moe
