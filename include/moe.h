/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts layer library.
 *
 * One MoE layer shaped like Kimi K3.1 (top-16 of 896 routed experts plus 2
 * always-on shared experts, MXFP4 SwiGLU experts) and the Q8_0 multi-row
 * spine matmul.  Source: "Run Kimi 3.1 locally on one GPU" (argonautlabs.ai)
 * and its sections named per function below.
 *
 * Conventions (all functions):
 *  - Every array pointer is DEVICE memory allocated and owned by the caller.
 *    The library never allocates, frees or retains caller memory.  Structs
 *    passed by pointer (moe_experts) are HOST memory, read during the call.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued on it; no function synchronises the device or the stream, and
 *    each returns as soon as its kernels are enqueued.
 *  - Return value: MOE_OK (0) or a negative moe_status.  Argument errors are
 *    detected on the host before anything is enqueued; then nothing is
 *    enqueued and no output is touched.
 *  - Arrays are row-major and densely packed.  Floating outputs are fp32.
 *  - M = 0 rows is valid and enqueues nothing.
 *  - Rows of one call never influence each other's results: the result of a
 *    row is bit-identical whether it is alone (M = 1) or inside a block of
 *    at most 16 rows, for every function here (the verification blocks of "A
 *    drafter that leaves the answer unchanged" must reproduce one-row steps
 *    exactly), and bit-identical across calls of any M for every function
 *    but the router logits: moe_route's logits in calls of more than 16 rows
 *    (a matrix-core form with another summation order) equal each other
 *    across such calls bit for bit and the one-row logits within rounding.
 *    Everything after the logits is bit-identical for the same logits.
 *
 * MXFP4 storage (OCP MX v1.0 elements; the byte layout is this library's
 * data contract, the pages give only the format name and the 17,547,264-byte
 * expert size, "One GPU, three storage tiers"):
 *  - a matrix [rows x K] (K a multiple of 32) is a codes plane of rows*K/2
 *    bytes, element 2i in the LOW nibble of byte i and element 2i+1 in the
 *    high nibble (E2M1: sign, 2-bit exponent with bias 1, 1-bit mantissa),
 *    followed by a scales plane of rows*K/32 E8M0 bytes (2^(b-127)), scale j
 *    of a row covering its elements 32j..32j+31;
 *  - an expert record is W_gate [f x d], W_up [f x d], W_down [d x f], each
 *    as codes plane then scales plane, back to back: 3*d*f*17/32 bytes
 *    (17,547,264 at d=7168, f=1536);
 *  - a layer is n_routed + n_shared records at a fixed stride; shared expert
 *    s has id n_routed + s.
 * E8M0 byte 255 (NaN) and bytes that would make a weight overflow fp32 are
 * outside the supported input range.
 *
 * Codes-plane order (moe_layout): the order above is MOE_LAYOUT_ROWS.  In
 * MOE_LAYOUT_TILES the blocks of 32 elements (16 bytes) of each codes plane
 * are permuted: block kb of row `row` sits at ((row/16)*(K/32) + kb)*256 +
 * (row%16)*16, so one 16-row tile's blocks lie side by side; scales planes
 * and record size are unchanged.  Every function gives bit-identical results
 * for the two orders; the tile order reads faster (each wave's load is one
 * contiguous kilobyte).  moe_pack_experts converts between them.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument: NULL pointer, negative size, k > E, d % 32, ... */
  MOE_EUNSUPPORTED = -2, /* valid but outside what this build implements (see per function) */
  MOE_EHIP = -3,         /* a HIP launch or runtime call failed */
  MOE_ESCRATCH = -4      /* moe_layer_mxfp4_noalloc: the call needs more than its static scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILES = 1 } moe_layout;

/* One layer's experts, resident in device memory. */
typedef struct {
  const uint8_t *base; /* device: (n_routed + n_shared) * stride bytes, 16-byte aligned */
  int64_t stride;      /* bytes between records, >= 3*d*f*17/32, multiple of 16 */
  int32_t d;           /* model width (reduction dim of gate/up), multiple of 32 */
  int32_t f;           /* expert FFN width, multiple of 32 */
  int32_t n_routed;    /* E */
  int32_t n_shared;    /* S, applied to every row with weight 1 */
  int32_t layout;      /* moe_layout of the codes planes */
} moe_experts;

/* Router ("Read the experts the router needs": top-k routing, k = 16 of
 * E = 896 in the Kimi layer).  The router function is softmax over the E
 * logits; the k largest are kept and their probabilities renormalised to
 * sum to 1.
 *
 *   x         [M x d] fp32 or bf16 (x_dtype), the layer input rows.
 *   w_router  [E x d] fp32.  If non-NULL, logits[m,e] = sum_c w_router[e,c]*x[m,c]
 *             is computed and written to `logits`.  If NULL, `logits` is an
 *             INPUT (x is then not read and may be NULL).
 *   logits    [M x E] fp32, output or input as above.
 *   topk_ids  [M x k] int32 out: expert ids in rank order (larger logit first,
 *             equal logits to the lower index, NaN ranks below every number).
 *   topk_w    [M x k] fp32 out: w[m,j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *             with l_0 the top logit (the renormalised softmax; summed in rank
 *             order).  Undefined (NaN) when the top logit is not finite.
 * Requires 1 <= k <= min(E, 64), E <= 4096, d % 32 == 0 (when w_router != NULL).
 */
int moe_route(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t d,
              int32_t E, int32_t k, int32_t *topk_ids, float *topk_w, void *stream);

/* Bucketing: group the M*(k+S) slots by expert so that one pass over an
 * expert's weights serves every row of the call that selected it ("A drafter
 * that leaves the answer unchanged": a block's weight traffic is one read per
 * distinct expert).  Slot t = m*(k+S)+j is routed expert topk_ids[m,j] for j < k and
 * shared expert E+(j-k) for j >= k.
 *
 *   offsets   [E+S+1] int32 out: exclusive prefix sum of per-expert slot
 *             counts; offsets[E+S] = M*(k+S).
 *   perm      [M*(k+S)] int32 out: slots sorted by (expert, slot), i.e. expert
 *             e's slots in ascending order at perm[offsets[e] .. offsets[e+1]).
 *   active    [E+S] int32 out: the experts with at least one slot, ascending,
 *             in active[0 .. *n_active).  Entries beyond are unspecified.
 *   n_active  [1] int32 out.
 *   dev_error [1] int32 out: set to 0, or to 1 if some topk_ids entry is
 *             outside [0,E) or a row repeats an expert.  Such slots are
 *             dropped; every write stays in bounds and the other outputs
 *             are unspecified.  Read after synchronising the stream.
 * Requires 1 <= k, E + S <= 4096.  All outputs are exact (integer).
 */
int moe_bucket(const int32_t *topk_ids, int32_t M, int32_t k, int32_t E, int32_t n_shared, int32_t *offsets,
               int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error, void *stream);

/* Expert FFN over the bucketed slots ("A drafter that leaves the answer
 * unchanged": one pass over an expert's weights per call, whatever the number
 * of its rows).  Experts are SwiGLU: y = W_down (silu(W_gate x) * (W_up x)),
 * silu(z) = z/(1+e^-z).
 *
 *   x         [M x d] fp32 or bf16 (x_dtype).
 *   M, k      as given to moe_bucket; S = W->n_shared.
 *   W         host pointer to the layer's expert table (device records).
 *   offsets, perm, active, n_active: moe_bucket's outputs for these M, k.
 *   y_slots   [M*(k+S) x d] fp32 out: row t holds slot t's expert output for
 *             row m = t/(k+S).  Every slot row is written.
 *   workspace device scratch of at least moe_workspace_bytes(M, k, W) bytes,
 *             owned by the caller; contents on entry do not matter.
 * The result of a slot does not depend on M, on the other rows, or on the
 * order of the active list.  Requires W->d % 32 == 0 and W->f % 32 == 0;
 * MOE_EUNSUPPORTED if a record, x or the workspace would exceed 2^30 bytes.
 */
int moe_expert_ffn_mxfp4(const void *x, moe_dtype x_dtype, int32_t M, int32_t k, const moe_experts *W,
                         const int32_t *offsets, const int32_t *perm, const int32_t *active,
                         const int32_t *n_active, float *y_slots, void *workspace, size_t workspace_bytes,
                         void *stream);

/* The two stages of moe_expert_ffn_mxfp4, for callers that time or schedule
 * them apart.  moe_ffn_gateup_mxfp4 computes h = silu(W_gate x) * (W_up x) for
 * every slot into the workspace; moe_ffn_down_mxfp4 then computes
 * y_slots = W_down h from it.  The down stage must follow the gate/up stage on
 * the same stream with the same M, k, W, bucketing arrays and workspace, with
 * nothing writing that workspace in between.  Together they enqueue exactly
 * what moe_expert_ffn_mxfp4 enqueues and give bit-identical y_slots.
 * Arguments, requirements and errors are those of moe_expert_ffn_mxfp4. */
int moe_ffn_gateup_mxfp4(const void *x, moe_dtype x_dtype, int32_t M, int32_t k, const moe_experts *W,
                         const int32_t *offsets, const int32_t *perm, const int32_t *active,
                         const int32_t *n_active, void *workspace, size_t workspace_bytes, void *stream);
int moe_ffn_down_mxfp4(int32_t M, int32_t k, const moe_experts *W, const int32_t *offsets, const int32_t *perm,
                       const int32_t *active, const int32_t *n_active, float *y_slots, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Copies n_records expert records (d, f, stride as in moe_experts) from src
 * to dst with their codes planes in order `to_layout` (src holds the other
 * order); scales planes and padding are copied unchanged.  src and dst are
 * distinct device buffers of n_records * stride bytes, 16-byte aligned.
 * Converting back gives the original bytes. */
int moe_pack_experts(const uint8_t *src, uint8_t *dst, int64_t n_records, int64_t stride, int32_t d, int32_t f,
                     moe_layout to_layout, void *stream);

/* Bytes of workspace moe_expert_ffn_mxfp4 needs for M rows (host-only query;
 * returns 0 for invalid arguments). */
size_t moe_workspace_bytes(int32_t M, int32_t k, const moe_experts *W);

/* Weighted combine: out[m,r] = sum_{j<k} topk_w[m,j] * y_slots[m*(k+S)+j, r]
 *                              + sum_{s<S} y_slots[m*(k+S)+k+s, r],
 * accumulated in fp32 in slot order (routed experts by the router's weights,
 * shared experts with weight 1).
 *   y_slots [M*(k+S) x d] fp32, topk_w [M x k] fp32, out [M x d] fp32.
 * Requires k >= 1, S >= 0, d % 4 == 0. */
int moe_combine(const float *y_slots, const float *topk_w, int32_t M, int32_t k, int32_t n_shared, int32_t d,
                float *out, void *stream);

/* One MoE layer in one call: moe_route, moe_bucket, moe_expert_ffn_mxfp4 and
 * moe_combine in that order ("Read the experts the router needs" and "A
 * drafter that leaves the answer unchanged").  Every
 * argument means what it means there, with E = W->n_routed and d = W->d, and
 * every output (logits when computed, topk_ids, topk_w, the bucketing
 * arrays, dev_error, y_slots, out) is bit-identical to what those four calls
 * give: the same kernels, enqueued by one call.
 *   workspace  at least moe_workspace_bytes(M, k, W) bytes; contents on
 *              entry do not matter; calls that share a workspace must not
 *              overlap (same stream, or ordered by events).
 * Requirements and errors are the union of the four functions'. */
int moe_layer_mxfp4(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M, int32_t k,
                    const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *perm,
                    int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* moe_layer_mxfp4 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It enqueues the same kernels and every
 * output is bit-identical to moe_layer_mxfp4's for the same arguments.
 *
 * Scratch: a static device array of moe_noalloc_scratch_bytes() (8 MiB) per
 * GPU, part of the library's code object; each GPU the library runs on holds
 * it until the process ends.  The first call on a device looks its address up
 * (with that device current); no call allocates or frees memory.  A call
 * whose scratch need (moe_workspace_bytes(M, k, W)) exceeds the array returns
 * MOE_ESCRATCH before enqueueing anything: a Kimi-shaped layer (d = 7168,
 * f = 1536, k = 16, S = 2) needs 1.77 MB at 16 rows and fits up to 75 rows.
 * The array keeps the last call's contents; no call relies on them (every
 * kernel writes what it reads first).  All calls on one GPU share the array,
 * so calls that may overlap on one GPU race: issue them on one stream, or
 * order them with events.  `stream` (or, for the null stream, the current
 * device) selects the GPU.  Other arguments, requirements and errors are
 * moe_layer_mxfp4's. */
int moe_layer_mxfp4_noalloc(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M,
                            int32_t k, const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                            int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots,
                            float *out, void *stream);
/* Bytes of the static scratch array of moe_layer_mxfp4_noalloc (host-only). */
size_t moe_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * Expert streaming ("One GPU, three storage tiers" and "Read the experts the
 * router needs": a device expert cache in front of a pinned host pool).
 * Experts in the device cache run immediately; the others are copied up from
 * the host pool over several streams and computed group by group as the
 * copies complete.
 * The disk tier of the pages is not modelled: the host pool holds every
 * expert of n_layers layers.
 *
 * Device pool slots (records of `stride` bytes):
 *   [0, n_layers*n_shared)            the shared experts, uploaded at creation
 *   next n_transient slots             experts used for one call only
 *   the rest (at least one)            cached experts, by (layer, expert)
 * Cache policy (also run on the host alone by moe_cache_simulate): the
 * experts of a call are taken in ascending id; those cached are hits.  With
 * admit_min_rows > 0 (the row-count admission rule of "A drafter that leaves
 * the answer unchanged"), a miss used by fewer rows
 * takes a transient slot while one is left.  Other misses are admitted into
 * the lowest free cached slot, else the least recently used cached slot
 * (lowest on equal age) not holding an expert of this call; with none left
 * they take transient slots. */
typedef struct moe_expert_cache moe_expert_cache; /* opaque, owned by the library */

typedef struct {
  void *device_pool;       /* device, n_slots * stride bytes, 16-byte aligned, caller-owned */
  int32_t n_slots;
  const void *host_pool;   /* PINNED host memory (hipHostMalloc, torch pin_memory), caller-owned:
                              n_layers * (n_routed + n_shared) records of `stride` bytes, layer
                              after layer, each layer laid out as moe_experts records */
  int32_t n_layers, n_routed, n_shared;
  int32_t d, f;            /* multiples of 32 */
  int64_t stride;          /* >= 3*d*f*17/32, multiple of 16 */
  int32_t n_upload_streams; /* 1..8 */
  int32_t upload_groups;   /* 1..16: misses are uploaded and computed in this many groups */
  int32_t admit_min_rows;  /* 0 = plain LRU */
  int32_t n_transient;     /* >= 0 */
  int32_t layout;          /* moe_layout of the host pool's records (kept in the device pool) */
} moe_cache_config;

typedef struct {
  int64_t calls, hits, misses, admitted, bytes_uploaded; /* routed experts only; since creation */
} moe_cache_stats;

/* Creates the cache: upload streams, events, small pinned and device plan
 * buffers (owned by the cache) and a synchronous upload of every shared
 * expert.  The pools stay owned by the caller and must outlive the cache.
 * MOE_EINVAL for a bad configuration or a host pool that is not pinned. */
int moe_cache_create(const moe_cache_config *cfg, moe_expert_cache **out);
/* Waits for the device to be idle, then frees what moe_cache_create made. */
int moe_cache_destroy(moe_expert_cache *cache);
int moe_cache_get_stats(const moe_expert_cache *cache, moe_cache_stats *stats);

/* moe_layer_mxfp4 for layer `layer` of the host pool, its experts streamed
 * into the device cache as needed.  Arguments and outputs are those of
 * moe_layer_mxfp4 (d, f, E, S from the configuration), and every output is
 * bit-identical to moe_layer_mxfp4 on the same layer held in device memory.
 * Unlike the other calls it SYNCHRONISES `stream` once, after the bucketing
 * (the experts to fetch are known only then), so it cannot be captured in a
 * graph.  Calls on one cache must come from one host thread on one stream.
 * MOE_EUNSUPPORTED if min(E, M*k) exceeds the transient plus cached slots.
 * Device pool offsets of a slot's record are 64-bit; a record itself is
 * addressed with 32-bit offsets (stride < 2^30). */
int moe_layer_streamed(moe_expert_cache *cache, int32_t layer, const void *x, moe_dtype x_dtype,
                       const float *w_router, float *logits, int32_t M, int32_t k, int32_t *topk_ids, float *topk_w,
                       int32_t *offsets, int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error,
                       float *y_slots, float *out, void *workspace, size_t workspace_bytes, void *stream);

/* The cache policy alone, on the host (no device call): n_calls calls, call
 * i of layer call_layer[i] with call_n[i] routed experts (ascending, distinct)
 * at experts[...] used by rows[...] rows each, concatenated over the calls.
 * Writes per entry its slot (0 .. n_transient-1 transient, then cached),
 * hit (0/1) and admitted (0/1).  MOE_EUNSUPPORTED if a call does not fit. */
int moe_cache_simulate(int32_t n_layers, int32_t n_routed, int32_t n_cache, int32_t n_transient,
                       int32_t admit_min_rows, int32_t n_calls, const int32_t *call_layer, const int32_t *call_n,
                       const int32_t *experts, const int32_t *rows, int32_t *slot, int32_t *hit, int32_t *admitted);

/* Q8_0 spine matmul ("A drafter that leaves the answer unchanged" and "One
 * GPU, three storage tiers": the spine is stored as Q8_0, and a call with up
 * to 8 rows reads each weight from HBM once rather than once per row):
 *   Y[m,n] = sum_c X[m,c] * Wq[n,c] * Ws[n, c/32]
 *   X  [M x K] fp32;  Wq [N x K] int8;  Ws [N x K/32] fp16 bit patterns;
 *   Y  [M x N] fp32 out.
 * Requires 1 <= M <= 8 (M = 0 enqueues nothing), K % 32 == 0, N >= 1. */
int q8_0_matmul(const float *X, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N, float *Y,
                void *stream);

/* q8_0_matmul with Wq in the given order.  MOE_LAYOUT_TILES (N % 16 == 0):
 * block b (32 bytes) of weight row n sits at ((n/16)*(K/32) + b)*512 +
 * (n%16)*32, so one step of a 16-row tile is one contiguous kilobyte; the
 * results are bit-identical to row order.  q8_0_pack converts Wq. */
int q8_0_matmul_layout(const float *X, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N,
                       float *Y, moe_layout layout, void *stream);

/* dst = the int8 plane [N x K] of src in order `to_layout` (src holds the
 * other order); N % 16 == 0, K % 32 == 0, distinct 16-byte aligned device
 * buffers.  The fp16 scales plane is the same in both orders. */
int q8_0_pack(const int8_t *src, int8_t *dst, int32_t N, int32_t K, moe_layout to_layout, void *stream);

/* ------------------------------------------------------------------------
 * Block verification ("A drafter that leaves the answer unchanged" and the
 * run record).  A harness over a stack of layers checks drafted tokens in one
 * multi-row block: a draft is accepted while it equals the greedy choice,
 * block rows must match one-row steps bit for bit, and every position's
 * logits are FNV-1a hashed on both sides.  The helpers below are exact. */

/* Rows of a Q8_0 matrix as fp32 (an embedding lookup):
 * X[m, c] = Wq[ids[m], c] * Ws[ids[m], c/32]; an id outside [0, N) gives a zero
 * row.  Wq in either order (tiles: N % 16 == 0).  X [M x K] 16-byte aligned,
 * Wq [N x K] 4-byte aligned, K % 32 == 0. */
int q8_0_rows(const int32_t *ids, int32_t M, int32_t K, const int8_t *Wq, const uint16_t *Ws, int32_t N, float *X,
              moe_layout layout, void *stream);

/* Residual update: if a != NULL, h[i] += a[i] (fp32); then, if h_bf16 != NULL,
 * h_bf16[i] = bf16 bits of h[i], rounded to nearest even.  n >= 0 elements. */
int moe_residual_bf16(float *h, const float *a, int64_t n, uint16_t *h_bf16, void *stream);

/* RMS normalisation per row, no gain: out[m,c] = h[m,c] / sqrt(mean_c h[m,c]^2 + eps)
 * (computed as h * (1 / sqrt(...)) in fp32, the sum of squares in an order
 * that depends only on d), written as fp32 to `out` and/or as bf16 bits
 * (nearest even) to `out_bf16` (either may be NULL, not both).  h [M x d];
 * h and out 16-byte aligned, out_bf16 8-byte aligned. */
int moe_rmsnorm(const float *h, int32_t M, int32_t d, float eps, float *out, uint16_t *out_bf16, void *stream);

/* Greedy choice per row: idx[m] = the index of the largest X[m, :], the lowest
 * index among equal values, NaN below every number.  X [M x N], 16-byte
 * aligned. */
int moe_argmax_rows(const float *X, int32_t M, int32_t N, int32_t *idx, void *stream);

/* hash[m] = 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime
 * 0x100000001b3) of the 4*N bytes of row m of X [M x N] fp32, in memory order.
 * A sequential recurrence: one thread per row, milliseconds for long rows. */
int moe_fnv1a_rows(const float *X, int32_t M, int32_t N, uint64_t *hash, void *stream);

/* One MX-scaled matrix-core instruction (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4),
 * the building block of an expert GEMM on MXFP4 weights without a bf16
 * decode ("What is established—and what remains open": expert GEMM choices
 * are an arithmetic path of their own).  The FFN kernels above do not use
 * it; this entry point exists so that its arithmetic can be measured:
 *   D[i][j] = sum_{k<128} A[i][k] sA[i][k/32] B[k][j] sB[j][k/32]
 * with the instruction's own summation and rounding, fp32 out.
 *   a_codes   [16 x 64] bytes: A row i, K 0..127 as E2M1 codes, element 2c
 *             in the low nibble of byte c (the MXFP4 codes layout above).
 *   a_scales  [16 x 4] E8M0 bytes: scale of row i, K block b (32 elements).
 *   b_codes   [16 x 128] bytes: B column j, K 0..127, one OCP FP8 E4M3 code
 *             per byte (bias 7, no infinities, 0x7F/0xFF NaN).
 *   b_scales  [16 x 4] E8M0 bytes: scale of column j, K block b.
 *   d         [16 x 16] fp32 out, row-major.
 * One wave on `stream`; a_codes and b_codes 16-byte aligned. */
int moe_mx_mfma_probe(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                      const uint8_t *b_scales, float *d, void *stream);

/* Human-readable name of a status code (static string). */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
