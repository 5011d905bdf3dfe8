// Bucketing: stable counting sort of the M*(k+S) slots by expert, so that
// the slots of one expert are contiguous and the FFN can serve them all from
// a single pass over that expert's weights ("Run Kimi 3.1 locally on one
// GPU", section "A drafter that leaves the answer unchanged").  One workgroup; every result is an integer and exact.
//
// Stable rank without sorting: within a row the k routed experts and the S
// shared experts are distinct, so the rank of slot (m, j) inside expert e's
// segment is the number of earlier rows that chose e.  Rows are taken 64 at a
// time; mask[e] has bit (m mod 64) set for each row of the chunk that chose
// e, and rank = base[e] + popcount(mask[e] & bits below m).
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr int BK_THREADS = 1024;
// Dynamic LDS of the general bucket kernel: its masks and counts, plus, when
// they fit, every slot's expert as an int16 (bucket_kernel, `cached`).
constexpr int kBkMaxLds = 152 * 1024;
// Dynamic LDS the fused top-k + bucket kernel may take: gfx950 gives a
// workgroup 160 KB in all, and the kernel holds about 4 KB of static LDS.
constexpr int kTbMaxLds = 152 * 1024;

// Expert of slot t, or -1 for a routed id outside [0, E).
__device__ __forceinline__ int slot_expert(const int32_t *ids, int t, int k, int kps, int E) {
  const int m = t / kps, j = t - m * kps;
  if (j >= k) return E + (j - k);
  const int e = ids[(int64_t)m * k + j];
  return (e >= 0 && e < E) ? e : -1;
}

// cached: the counting pass also keeps each slot's expert in LDS (-1 for an
// id outside [0, E)), so the placement rounds read no global memory; the
// results are the same integers either way.
__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(const int32_t *__restrict__ ids, int M, int k, int E,
                                                            int S, int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ perm, int32_t *__restrict__ active,
                                                            int32_t *__restrict__ n_active,
                                                            int32_t *__restrict__ dev_error, int cached) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int NE = E + S;
  unsigned long long *mask = (unsigned long long *)smem;  // [NE]
  int32_t *base = (int32_t *)(mask + NE);                 // [NE] counts, then running bases
  int16_t *eid = (int16_t *)(base + NE);                  // [T] when cached
  __shared__ int32_t wave_sum[16][2];
  __shared__ int32_t err;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kps = k + S;
  const int T = M * kps;

  for (int e = tid; e < NE; e += BK_THREADS) base[e] = 0;
  if (tid == 0) err = 0;
  __syncthreads();
  // ---- counts
  for (int t = tid; t < T; t += BK_THREADS) {
    const int e = slot_expert(ids, t, k, kps, E);
    if (cached) eid[t] = (int16_t)e;
    if (e < 0 || e >= NE) err = 1;
    else atomicAdd(&base[e], 1);
  }
  __syncthreads();
  // ---- exclusive scan of counts (offsets) and of nonempty flags (active)
  const int per = (NE + BK_THREADS - 1) / BK_THREADS;
  const int e_beg = tid * per;
  int c_loc = 0, a_loc = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e_beg + i;
    if (e < NE) { c_loc += base[e]; a_loc += base[e] > 0; }
  }
  int cv = c_loc, av = a_loc;
  for (int o = 1; o < 64; o <<= 1) {
    const int tc = __shfl_up(cv, o, 64), ta = __shfl_up(av, o, 64);
    if (lane >= o) { cv += tc; av += ta; }
  }
  if (lane == 63) { wave_sum[wv][0] = cv; wave_sum[wv][1] = av; }
  __syncthreads();
  int c_ex = cv - c_loc, a_ex = av - a_loc, c_tot = 0, a_tot = 0;
  for (int w2 = 0; w2 < BK_THREADS / 64; ++w2) {
    if (w2 < wv) { c_ex += wave_sum[w2][0]; a_ex += wave_sum[w2][1]; }
    c_tot += wave_sum[w2][0];
    a_tot += wave_sum[w2][1];
  }
  __syncthreads();  // every thread has read its counts range before it is overwritten
  for (int i = 0; i < per; ++i) {
    const int e = e_beg + i;
    if (e < NE) {
      const int c = base[e];
      offsets[e] = c_ex;
      if (c > 0) active[a_ex++] = e;
      base[e] = c_ex;
      mask[e] = 0ull;
      c_ex += c;
    }
  }
  if (tid == 0) {
    offsets[NE] = c_tot;
    *n_active = a_tot;
  }
  __syncthreads();
  // ---- stable placement, 64 rows at a time (the masks start at zero and
  // each round clears them as it adds them to the bases)
  for (int m0 = 0; m0 < M; m0 += 64) {
    const int mrows = (M - m0) < 64 ? (M - m0) : 64;
    const int tc = mrows * kps;
    for (int i = tid; i < tc; i += BK_THREADS) {
      const int t = m0 * kps + i;
      const int e = cached ? (int)eid[t] : slot_expert(ids, t, k, kps, E);
      if (e >= 0 && e < NE) {
        const unsigned long long bit = 1ull << (t / kps - m0);
        const unsigned long long old = atomicOr(&mask[e], bit);
        if (old & bit) err = 1;  // a row names the same expert twice
      }
    }
    __syncthreads();
    for (int i = tid; i < tc; i += BK_THREADS) {
      const int t = m0 * kps + i;
      const int e = cached ? (int)eid[t] : slot_expert(ids, t, k, kps, E);
      if (e >= 0 && e < NE) {
        const unsigned long long bit = 1ull << (t / kps - m0);
        const int rank = base[e] + __popcll(mask[e] & (bit - 1ull));
        if (rank < T) perm[rank] = t;
      }
    }
    __syncthreads();
    for (int e = tid; e < NE; e += BK_THREADS) {
      base[e] += __popcll(mask[e]);
      mask[e] = 0ull;
    }
    __syncthreads();
  }
  if (tid == 0) *dev_error = err;
}

// Small batches (T <= threads of the workgroup, M <= 64 rows): one thread
// per slot keeps its expert in a register (e_mine: the expert, -1 for a
// routed id outside [0, E), -2 for a thread without a slot), so the ids are
// read once; the counts and the 64-row occupancy masks are built in the same
// pass, and the arithmetic of every output is the general kernel's.  Every
// thread of the workgroup calls it (it has barriers).  smem: NE 64-bit masks
// then NE int32 counts; wave_sum: one pair per wave.
__device__ __forceinline__ void bucket_small_body(int e_mine, int M, int kps, int NE, int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ perm, int32_t *__restrict__ active,
                                                  int32_t *__restrict__ n_active, int32_t *__restrict__ dev_error,
                                                  uint8_t *smem, int32_t (*wave_sum)[2], int32_t *err) {
  unsigned long long *mask = (unsigned long long *)smem;  // [NE]
  int32_t *base = (int32_t *)(mask + NE);                 // [NE] counts, then bases
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nth = blockDim.x, nw = nth >> 6;
  const int T = M * kps;
  for (int e = tid; e < NE; e += nth) {
    base[e] = 0;
    mask[e] = 0ull;
  }
  if (tid == 0) *err = 0;
  __syncthreads();
  const unsigned long long bit = 1ull << (tid < T ? tid / kps : 0);
  if (e_mine == -1) *err = 1;
  if (e_mine >= 0) {
    atomicAdd(&base[e_mine], 1);
    const unsigned long long old = atomicOr(&mask[e_mine], bit);
    if (old & bit) *err = 1;  // a row names the same expert twice
  }
  __syncthreads();
  // exclusive scans of the counts (offsets) and of the nonempty flags (active)
  const int per = (NE + nth - 1) / nth;
  const int e_beg = tid * per;
  int c_loc = 0, a_loc = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e_beg + i;
    if (e < NE) { c_loc += base[e]; a_loc += base[e] > 0; }
  }
  int cv = c_loc, av = a_loc;
  for (int o = 1; o < 64; o <<= 1) {
    const int tc = __shfl_up(cv, o, 64), ta = __shfl_up(av, o, 64);
    if (lane >= o) { cv += tc; av += ta; }
  }
  if (lane == 63) { wave_sum[wv][0] = cv; wave_sum[wv][1] = av; }
  __syncthreads();
  int c_ex = cv - c_loc, a_ex = av - a_loc, c_tot = 0, a_tot = 0;
  for (int w2 = 0; w2 < nw; ++w2) {
    if (w2 < wv) { c_ex += wave_sum[w2][0]; a_ex += wave_sum[w2][1]; }
    c_tot += wave_sum[w2][0];
    a_tot += wave_sum[w2][1];
  }
  __syncthreads();  // every count is read before it becomes a base
  for (int i = 0; i < per; ++i) {
    const int e = e_beg + i;
    if (e < NE) {
      const int c = base[e];
      offsets[e] = c_ex;
      if (c > 0) active[a_ex++] = e;
      base[e] = c_ex;
      c_ex += c;
    }
  }
  if (tid == 0) {
    offsets[NE] = c_tot;
    *n_active = a_tot;
  }
  __syncthreads();
  if (e_mine >= 0) {
    const int rank = base[e_mine] + __popcll(mask[e_mine] & (bit - 1ull));
    if (rank < T) perm[rank] = tid;
  }
  __syncthreads();
  if (tid == 0) *dev_error = *err;
}

__global__ __launch_bounds__(BK_THREADS) void bucket_small_kernel(const int32_t *__restrict__ ids, int M, int k, int E,
                                                                  int S, int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ perm,
                                                                  int32_t *__restrict__ active,
                                                                  int32_t *__restrict__ n_active,
                                                                  int32_t *__restrict__ dev_error) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int32_t wave_sum[BK_THREADS / 64][2];
  __shared__ int32_t err;
  const int tid = threadIdx.x, kps = k + S;
  const int e_mine = tid < M * kps ? slot_expert(ids, tid, k, kps, E) : -2;
  bucket_small_body(e_mine, M, kps, E + S, offsets, perm, active, n_active, dev_error, smem, wave_sum, &err);
}

// ------------------------------------------------------------------ top-k + bucket
// A few rows (M <= 4, k + S <= 64): one workgroup of M waves; wave m ranks
// row m (topk_row: the top-k kernel's arithmetic), the ids go to LDS, and
// then every thread takes slot `tid` (T = M (k+S) <= 64 M) and the workgroup
// buckets them (bucket_small_body).  Same results as topk_kernel followed by
// bucket_small_kernel, in one launch.  Dynamic LDS: the ranking lists of the
// M waves, then (reused) the bucket's masks and counts.  Measured on MI355X
// at the Kimi shape: the 1- and 2-row layers gain about 1 us; at 16 rows the
// 16 rankings on one CU take longer than the separate top-k kernel's 4 CUs
// and the layer loses 5 us, hence the limit.
constexpr int TB_MAX_ROWS = 4;

template <int NPL>
__global__ __launch_bounds__(TB_MAX_ROWS * 64) void topk_bucket_kernel(
    const float *__restrict__ logits, int M, int E, int k, int S, int32_t *__restrict__ ids, float *__restrict__ w,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active, int32_t *__restrict__ dev_error) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int32_t wave_sum[TB_MAX_ROWS][2];
  __shared__ int32_t err;
  __shared__ int32_t sids[TB_MAX_ROWS * 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t id;
  float wt;
  topk_row_any<NPL>(logits + (int64_t)wv * E, E, k, (uint64_t(*)[64])(smem + (size_t)wv * topk_wave_lds(NPL)), lane, id,
                wt);
  if (lane < k) {
    ids[(int64_t)wv * k + lane] = id;
    w[(int64_t)wv * k + lane] = wt;
  }
  const int kps = k + S, NE = E + S;
  // One row (the workgroup is one wave): bucket_one_row, same results as
  // the general path below.
  if (M == 1 && NE + 1 <= 64 * 64 && __ballot(lane < k && (id < 0 || id >= E)) == 0ull) {
    bucket_one_row(id, lane, E, k, S, offsets, perm, active, n_active, dev_error);
    return;
  }
  if (lane < k) sids[wv * k + lane] = id;
  __syncthreads();  // the ids are in LDS and every wave is done with its lists
  int e_mine = -2;
  if (tid < M * kps) {
    const int m = tid / kps, j = tid - m * kps;
    if (j >= k) {
      e_mine = E + (j - k);
    } else {
      const int e = sids[m * k + j];
      e_mine = (e >= 0 && e < E) ? e : -1;
    }
  }
  bucket_small_body(e_mine, M, kps, NE, offsets, perm, active, n_active, dev_error, smem, wave_sum, &err);
}

template <int NPL>
static int launch_topk_bucket(const float *logits, int M, int E, int k, int S, int32_t *ids, float *w,
                              int32_t *offsets, int32_t *perm, int32_t *active, int32_t *n_active,
                              int32_t *dev_error, size_t smem, hipStream_t stream) {
  static const bool lds_ok =
      hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_bucket_kernel<NPL>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kTbMaxLds) == hipSuccess;
  if (!lds_ok) {
    (void)hipGetLastError();  // leave no error behind for the next launch check
    return -3;
  }
  hipLaunchKernelGGL(topk_bucket_kernel<NPL>, dim3(1), dim3(M * 64), smem, stream, logits, M, E, k, S, ids, w,
                     offsets, perm, active, n_active, dev_error);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int bucket_launch(const int32_t *ids, int M, int k, int E, int S, int32_t *offsets, int32_t *perm, int32_t *active,
                  int32_t *n_active, int32_t *dev_error, hipStream_t stream) {
  const int NE = E + S;
  const size_t smem = (size_t)NE * (sizeof(unsigned long long) + sizeof(int32_t));
  if ((int64_t)M * (k + S) <= BK_THREADS && M <= 64)
    hipLaunchKernelGGL(bucket_small_kernel, dim3(1), dim3(BK_THREADS), smem, stream, ids, M, k, E, S, offsets, perm,
                       active, n_active, dev_error);
  else {
    // the slots' experts as int16 in LDS where they fit (NE <= 4096 fits int16)
    static const bool big_lds = hipFuncSetAttribute(reinterpret_cast<const void *>(&bucket_kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, kBkMaxLds) == hipSuccess;
    if (!big_lds) (void)hipGetLastError();  // leave no error behind for the launch check
    const size_t lim = big_lds ? (size_t)kBkMaxLds : (size_t)64 * 1024;
    const size_t with_ids = smem + (size_t)M * (k + S) * sizeof(int16_t);
    const int cached = with_ids <= lim ? 1 : 0;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(BK_THREADS), cached ? with_ids : smem, stream, ids, M, k, E, S,
                       offsets, perm, active, n_active, dev_error, cached);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int route_bucket_launch(const void *x, int x_bf16, const float *w_router, float *logits, int M, int d, int E, int k,
                        int S, int32_t *ids, float *w, int32_t *offsets, int32_t *perm, int32_t *active,
                        int32_t *n_active, int32_t *dev_error, hipStream_t stream) {
  if (w_router && logits_launch(x, x_bf16, w_router, logits, M, d, E, stream)) return -3;
  const int npl = (E + 63) / 64;
  const size_t lists = (size_t)M * topk_wave_lds(npl), bk = (size_t)(E + S) * (sizeof(unsigned long long) + 4);
  const size_t smem = lists > bk ? lists : bk;
  if (M <= TB_MAX_ROWS && k <= 64 && k + S <= 64 && smem <= (size_t)kTbMaxLds) {
    if (npl <= 1) return launch_topk_bucket<1>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 2) return launch_topk_bucket<2>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 4) return launch_topk_bucket<4>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 8) return launch_topk_bucket<8>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 14) return launch_topk_bucket<14>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 16) return launch_topk_bucket<16>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
    if (npl <= 32) return launch_topk_bucket<32>(logits, M, E, k, S, ids, w, offsets, perm, active, n_active, dev_error, smem, stream);
  }
  if (topk_launch(logits, M, E, k, ids, w, stream)) return -3;
  return bucket_launch(ids, M, k, E, S, offsets, perm, active, n_active, dev_error, stream);
}

// ------------------------------------------------------------------ combine
// out[m,r] = sum_{j<k} w[m,j] y[m*(k+S)+j, r] + sum_{s<S} y[m*(k+S)+k+s, r],
// fp32, in slot order.  One thread per 4 consecutive r; the slot rows are
// loaded CH at a time before their (ordered) accumulation, CH chosen so that
// k + S slots take one round of loads where it fits (18 at the Kimi shape).
constexpr int CB_THREADS = 64;
template <int CH>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                             int M, int k, int S, int d, float *__restrict__ out) {
  const int d4 = d >> 2;
  const int64_t idx = (int64_t)blockIdx.x * CB_THREADS + threadIdx.x;
  if (idx >= (int64_t)M * d4) return;
  const int64_t m = idx / d4;
  const int c = (int)(idx - m * d4) * 4;
  const int kps = k + S;
  const float *ym = y + m * kps * (int64_t)d + c;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < kps; j0 += CH) {
    f32x4 v[CH];
    float wj[CH];
    // clamped (always valid) indices: every load is issued, none waits on another
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int j = j0 + u;
      v[u] = *(const f32x4 *)(ym + (int64_t)(j < kps ? j : kps - 1) * d);
      wj[u] = w[m * k + (j < k ? j : k - 1)];
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int j = j0 + u;
      if (j < k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(wj[u], v[u][i], acc[i]);
      } else if (j < kps) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[u][i];
      }
    }
  }
  *(f32x4 *)(out + m * (int64_t)d + c) = acc;
}

int combine_launch(const float *y, const float *w, int M, int k, int S, int d, float *out, hipStream_t stream) {
  const int64_t n = (int64_t)M * (d / 4);
  const int64_t grid = (n + CB_THREADS - 1) / CB_THREADS;
  const int kps = k + S;
  if (kps <= 4)
    hipLaunchKernelGGL(combine_kernel<4>, dim3((unsigned)grid), dim3(CB_THREADS), 0, stream, y, w, M, k, S, d, out);
  else if (kps <= 9)
    hipLaunchKernelGGL(combine_kernel<9>, dim3((unsigned)grid), dim3(CB_THREADS), 0, stream, y, w, M, k, S, d, out);
  else
    hipLaunchKernelGGL(combine_kernel<18>, dim3((unsigned)grid), dim3(CB_THREADS), 0, stream, y, w, M, k, S, d, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace moe
