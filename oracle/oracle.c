/*
 * CPU oracle for one mixture-of-experts layer with MXFP4 experts and for the
 * Q8_0 multi-row spine matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * GPU path: every value below is written out from its definition.
 *
 * Sources ("Run Kimi 3.1 locally on one GPU", argonautlabs.ai):
 *   - section "Read the experts the router needs": the Kimi layer routes each
 *     token to k = 16 of its E = 896 experts;
 *   - section "A drafter that leaves the answer unchanged": verification
 *     blocks of up to 16 rows, whose per-row results must equal those of
 *     one-row steps bit for bit (so each row's result here is computed on its
 *     own, whatever block it sits in);
 *   - section "One GPU, three storage tiers": each expert is an MXFP4 record
 *     of 17,547,264 bytes, and the spine's matrices are stored as Q8_0.
 * The pages give neither the router function, the bit layout of MXFP4 or
 * Q8_0, nor any worked numeric example.  The readings used here (softmax,
 * top-k by logit with ties to the lower index, renormalised weights, SwiGLU
 * experts, low-nibble-first E2M1 codes with a plane of E8M0 scales, Q8_0 as an
 * int8 plane plus an fp16 scale per 32) are stated per function.
 *
 * Arithmetic: every floating-point result is accumulated in double precision
 * in the plain order of its definition (ascending reduction index) and
 * rounded once to fp32 where the layer stores a tensor.  Each output element
 * is computed by one thread, so results do not depend on the thread count.
 *
 * Parity status: every function here is pinned by a test that does not
 * re-derive it (closed forms, exhaustive tables, brute force, special cases);
 * the Kimi-sized real-valued outputs themselves have no printed value on the
 * pages and rest on those pins.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* Threads a parallel region of this library uses (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the threads later parallel regions use (no effect without OpenMP).
 * Results do not depend on it: every output element is one thread's. */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element formats                                                          */
/* ------------------------------------------------------------------------ */

/* E2M1 (OCP Microscaling Formats v1.0, FP4 element): bit 3 sign, bits 2..1
 * exponent with bias 1, bit 0 mantissa.  Exponent field 0 is subnormal:
 * value = m * 2^-1 * ... = 0.5*m.  Otherwise value = 2^(e-1) * (1 + m/2). */
double orc_e2m1(int code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
  return sign ? -mag : mag;
}

/* E8M0 (OCP MX v1.0 shared scale): 2^(b-127); 0xFF encodes NaN. */
double orc_e8m0(int b) {
  if (b == 255) return NAN;
  return ldexp(1.0, b - 127);
}

/* OCP FP8 E4M3 (an OCP MX v1.0 element type): sign, 4-bit exponent with bias
 * 7, 3-bit mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F and 0xFF are
 * NaN; there are no infinities (the largest value is 448). */
double orc_e4m3(int code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* One MX-scaled matrix tile, 16 x 16 over K = 128, the arithmetic of an
 * expert GEMM on MXFP4 weights with FP8 activations ("What is
 * established—and what remains open": expert GEMM choices are an arithmetic
 * path of their own):
 *   D[i][j] = sum_k A[i][k] sA[i][k/32] * B[k][j] sB[j][k/32]
 * A row i: 64 bytes of E2M1 codes (element 2c in the low nibble of byte c);
 * B column j: 128 bytes of E4M3 codes; scales: 4 E8M0 bytes per row/column.
 * The sum runs over ascending k in double precision. */
int orc_mx_tile(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes, const uint8_t *b_scales,
                double *d) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !d) return ORC_EINVAL;
  for (int i = 0; i < 16; ++i)
    for (int j = 0; j < 16; ++j) {
      double s = 0.0;
      for (int k = 0; k < 128; ++k) {
        const int byte = a_codes[i * 64 + k / 2];
        const double a = orc_e2m1((k & 1) ? (byte >> 4) : (byte & 15)) * orc_e8m0(a_scales[i * 4 + k / 32]);
        const double b = orc_e4m3(b_codes[j * 128 + k]) * orc_e8m0(b_scales[j * 4 + k / 32]);
        s += a * b;
      }
      d[i * 16 + j] = s;
    }
  return ORC_OK;
}

/* IEEE binary16 bits to double, written out from the format definition. */
double orc_fp16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return sign ? -v : v;
}

/* bfloat16 bits to float: the upper half of an IEEE binary32. */
void orc_widen_bf16(const uint16_t *src, int64_t n, float *dst) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)src[i] << 16;
    memcpy(&dst[i], &u, 4);
  }
}

/* ------------------------------------------------------------------------ */
/* MXFP4 matrices and the expert record                                     */
/* ------------------------------------------------------------------------ */

/* One MXFP4 matrix [rows x K], K a multiple of 32: a plane of codes, rows x K/2
 * bytes with element 2i in the low nibble of byte i and element 2i+1 in the
 * high nibble, then a plane of E8M0 scales, rows x K/32 bytes, scale j of a
 * row covering elements 32j..32j+31. */
static double mx_elem(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t r, int64_t c) {
  uint8_t byte = codes[r * (K / 2) + c / 2];
  int code = (c & 1) ? (byte >> 4) : (byte & 15);
  return orc_e2m1(code) * orc_e8m0(scales[r * (K / 32) + c / 32]);
}

/* Byte offsets of the six sections of one expert (gate codes, gate scales,
 * up codes, up scales, down codes, down scales) and the record size, for
 * model width d and FFN width f.  Gate and up are [f x d]; down is [d x f].
 * The page states 17,547,264 bytes per expert at d=7168, f=1536, which is
 * 3*d*f/32 blocks of 16 code bytes plus one scale byte. */
int orc_expert_layout(int64_t d, int64_t f, int64_t *off /* [7] */) {
  if (d <= 0 || f <= 0 || d % 32 || f % 32) return ORC_EINVAL;
  int64_t codes_gu = f * d / 2, scales_gu = f * d / 32;
  int64_t codes_dn = d * f / 2, scales_dn = d * f / 32;
  off[0] = 0;
  off[1] = off[0] + codes_gu;
  off[2] = off[1] + scales_gu;
  off[3] = off[2] + codes_gu;
  off[4] = off[3] + scales_gu;
  off[5] = off[4] + codes_dn;
  off[6] = off[5] + scales_dn; /* record size */
  return ORC_OK;
}

/* Dequantise a whole MXFP4 matrix to double (used by the pins only). */
int orc_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, double *out) {
  if (K % 32) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < K; ++c) out[r * K + c] = mx_elem(codes, scales, K, r, c);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Router                                                                   */
/* ------------------------------------------------------------------------ */

/* logits[m,e] = sum_c W_r[e,c] * x[m,c]  (W_r row-major [E x d]). */
int orc_router_logits(const float *x, const float *w_r, int32_t M, int32_t d, int32_t E, float *logits) {
  if (M < 0 || d <= 0 || E <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * E; ++i) {
    int64_t m = i / E, e = i % E;
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += (double)w_r[e * d + c] * (double)x[m * d + c];
    logits[i] = (float)s;
  }
  return ORC_OK;
}

/* Rank key: NaN ranks as -infinity. */
static double rank_val(float v) { return isnan(v) ? -INFINITY : (double)v; }

/* a ranks before b: larger logit first, equal logits by lower index. */
static int ranks_before(const float *row, int a, int b) {
  double va = rank_val(row[a]), vb = rank_val(row[b]);
  if (va != vb) return va > vb;
  return a < b;
}

/* Top-k and routing weights for each row.
 * The router is softmax over all E logits; the k experts with the largest
 * probability are selected (ranking by logit is the same order because exp is
 * increasing; equal logits go to the lower index; NaN ranks last), and the k
 * selected probabilities are renormalised to sum to one.  ids[m,0..k-1] are in
 * rank order and w[m,j] belongs to ids[m,j]. */
int orc_topk(const float *logits, int32_t M, int32_t E, int32_t k, int32_t *ids, float *w) {
  if (M < 0 || E <= 0 || k < 1 || k > E) return ORC_EINVAL;
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t m = 0; m < M; ++m) {
    const float *row = logits + m * E;
    int32_t *id = ids + m * k;
    char *taken = (char *)calloc((size_t)E, 1);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    if (!taken || !p) { err |= 1; free(taken); free(p); continue; }
    /* selection: k passes of "best remaining" */
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || ranks_before(row, e, best))) best = e;
      taken[best] = 1;
      id[j] = best;
    }
    /* softmax over all experts (max-shifted), NaN contributes probability 0 */
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e) if (rank_val(row[e]) > mx) mx = rank_val(row[e]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) { p[e] = exp(rank_val(row[e]) - mx); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    double ps = 0.0;
    for (int j = 0; j < k; ++j) ps += p[id[j]];
    for (int j = 0; j < k; ++j) w[m * k + j] = (float)(p[id[j]] / ps);
    free(taken);
    free(p);
  }
  return err ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Bucketing                                                                */
/* ------------------------------------------------------------------------ */

/* Slots t = m*(k+S)+j of M rows: j<k is routed expert ids[m,j]; j>=k is shared
 * expert E+(j-k), applied to every row.  Group the slots by expert so that
 * each expert's slots are contiguous (so one pass over its weights can serve
 * all of them): offsets[e]..offsets[e+1] is expert e's segment of perm,
 * perm lists slot indices ordered by (expert, slot), active lists the experts
 * with a nonempty segment in ascending order.  Returns ORC_EINVAL (and writes
 * nothing) when an id is outside [0,E). */
int orc_bucket(const int32_t *ids, int32_t M, int32_t k, int32_t E, int32_t S, int32_t *offsets, int32_t *perm,
               int32_t *active, int32_t *n_active) {
  if (M < 0 || k < 1 || E <= 0 || S < 0) return ORC_EINVAL;
  int64_t T = (int64_t)M * (k + S);
  int32_t NE = E + S;
  for (int64_t i = 0; i < (int64_t)M * k; ++i)
    if (ids[i] < 0 || ids[i] >= E) return ORC_EINVAL;
  int32_t *expert_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!expert_of) return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t) {
    int64_t m = t / (k + S), j = t % (k + S);
    expert_of[t] = (j < k) ? ids[m * k + j] : E + (int32_t)(j - k);
  }
  /* counts, then exclusive prefix sum */
  for (int32_t e = 0; e <= NE; ++e) offsets[e] = 0;
  for (int64_t t = 0; t < T; ++t) offsets[expert_of[t] + 1]++;
  for (int32_t e = 0; e < NE; ++e) offsets[e + 1] += offsets[e];
  /* stable placement: walk slots in ascending order */
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)NE);
  if (!fill) { free(expert_of); return ORC_EINVAL; }
  for (int32_t e = 0; e < NE; ++e) fill[e] = offsets[e];
  for (int64_t t = 0; t < T; ++t) perm[fill[expert_of[t]]++] = (int32_t)t;
  int32_t na = 0;
  for (int32_t e = 0; e < NE; ++e)
    if (offsets[e + 1] > offsets[e]) active[na++] = e;
  *n_active = na;
  free(fill);
  free(expert_of);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN (SwiGLU)                                                       */
/* ------------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y[n] = W_down * (silu(W_gate * x[n]) .* (W_up * x[n])) for rows x[0..nrows-1]
 * (each [d]) through one expert record (layout of orc_expert_layout).  Each
 * output element is an ascending-index sum of its own; handling several rows
 * per call only lets a weight element be decoded once for all of them.
 * Results rounded to fp32. */
int orc_expert_ffn(const float *x, int32_t nrows, const uint8_t *expert, int32_t d, int32_t f, float *y) {
  int64_t off[7];
  if (nrows < 0 || orc_expert_layout(d, f, off)) return ORC_EINVAL;
  if (nrows == 0) return ORC_OK;
  const uint8_t *gc = expert + off[0], *gs = expert + off[1];
  const uint8_t *uc = expert + off[2], *us = expert + off[3];
  const uint8_t *dc = expert + off[4], *ds = expert + off[5];
  double *h = (double *)malloc(sizeof(double) * (size_t)f * (size_t)nrows);
  if (!h) return ORC_EINVAL;
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t i = 0; i < f; ++i) {
    double *g = (double *)calloc((size_t)nrows * 2, sizeof(double));
    if (!g) { err |= 1; continue; }
    double *u = g + nrows;
    for (int64_t c = 0; c < d; ++c) {
      double wg = mx_elem(gc, gs, d, i, c), wu = mx_elem(uc, us, d, i, c);
      for (int64_t n = 0; n < nrows; ++n) {
        g[n] += wg * (double)x[n * d + c];
        u[n] += wu * (double)x[n * d + c];
      }
    }
    for (int64_t n = 0; n < nrows; ++n) h[n * f + i] = silu(g[n]) * u[n];
    free(g);
  }
  if (err) { free(h); return ORC_EINVAL; }
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t r = 0; r < d; ++r) {
    double *s = (double *)calloc((size_t)nrows, sizeof(double));
    if (!s) { err |= 1; continue; }
    for (int64_t i = 0; i < f; ++i) {
      double wd = mx_elem(dc, ds, f, r, i);
      for (int64_t n = 0; n < nrows; ++n) s[n] += wd * h[n * f + i];
    }
    for (int64_t n = 0; n < nrows; ++n) y[n * d + r] = (float)s[n];
    free(s);
  }
  free(h);
  return err ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                  */
/* ------------------------------------------------------------------------ */

/* out[m,r] = sum_{j<k} w[m,j] * y[m*(k+S)+j, r] + sum_{s<S} y[m*(k+S)+k+s, r]:
 * the routed experts weighted by the router, shared experts with weight one. */
int orc_combine(const float *y_slots, const float *w, int32_t M, int32_t k, int32_t S, int32_t d, float *out) {
  if (M < 0 || k < 1 || S < 0 || d <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * d; ++i) {
    int64_t m = i / d, r = i % d;
    double s = 0.0;
    for (int64_t j = 0; j < k; ++j) s += (double)w[m * k + j] * (double)y_slots[(m * (k + S) + j) * d + r];
    for (int64_t j = 0; j < S; ++j) s += (double)y_slots[(m * (k + S) + k + j) * d + r];
    out[i] = (float)s;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Q8_0 spine matmul                                                         */
/* ------------------------------------------------------------------------ */

/* Y[m,n] = sum_c X[m,c] * q[n,c] * s[n, c/32]: W stored as an int8 plane [N x K]
 * and an fp16 scale plane [N x K/32]. */
int orc_q8_0_matmul(const float *X, int32_t M, int32_t K, const int8_t *wq, const uint16_t *ws, int32_t N, float *Y) {
  if (M < 0 || K <= 0 || K % 32 || N <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * N; ++i) {
    int64_t m = i / N, n = i % N;
    double s = 0.0;
    for (int64_t c = 0; c < K; ++c)
      s += (double)X[m * K + c] * ((double)wq[n * K + c] * orc_fp16(ws[n * (K / 32) + c / 32]));
    Y[i] = (float)s;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* fp32-accumulation variants                                               */
/* ------------------------------------------------------------------------ */
/* The same definitions with every sum kept in fp32, in the order the layer's
 * specification states for an fp32-accumulating reference: a reduction over K
 * is cut into blocks of 32 consecutive indices; inside a block the terms are
 * added one after another in fp32 (each product rounded to fp32, then the
 * add), and the block partials are then added in ascending block order.
 * silu and the routing softmax use the fp32 expf.  The fp64 functions above
 * are the default reference (a tighter one: their only rounding is the final
 * store); these exist so the two readings can be compared.  The product is
 * compiled without contraction, so no multiply-add is fused. */

static float blocked_dot_f32(const float *a, const float *b, int64_t K) {
  float s = 0.0f;
  for (int64_t c0 = 0; c0 < K; c0 += 32) {
    float p = 0.0f;
    int64_t c1 = c0 + 32 < K ? c0 + 32 : K;
    for (int64_t c = c0; c < c1; ++c) {
      float t = a[c] * b[c];
      p = p + t;
    }
    s = s + p;
  }
  return s;
}

int orc_router_logits_f32(const float *x, const float *w_r, int32_t M, int32_t d, int32_t E, float *logits) {
  if (M < 0 || d <= 0 || E <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * E; ++i) {
    int64_t m = i / E, e = i % E;
    logits[i] = blocked_dot_f32(w_r + e * d, x + m * d, d);
  }
  return ORC_OK;
}

/* Top-k as orc_topk (same selection); weights w_j = expf(l_j - l_0) /
 * sum_{i<k} expf(l_i - l_0) in fp32 with l_0 the top logit, the normaliser
 * summed in rank order.  NaN logits are never selected before a number. */
int orc_topk_f32(const float *logits, int32_t M, int32_t E, int32_t k, int32_t *ids, float *w) {
  if (M < 0 || E <= 0 || k < 1 || k > E) return ORC_EINVAL;
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t m = 0; m < M; ++m) {
    const float *row = logits + m * E;
    int32_t *id = ids + m * k;
    char *taken = (char *)calloc((size_t)E, 1);
    if (!taken) { err |= 1; continue; }
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || ranks_before(row, e, best))) best = e;
      taken[best] = 1;
      id[j] = best;
    }
    float l0 = row[id[0]];
    float z = 0.0f;
    for (int j = 0; j < k; ++j) z = z + expf(row[id[j]] - l0);
    for (int j = 0; j < k; ++j) w[m * k + j] = expf(row[id[j]] - l0) / z;
    free(taken);
  }
  return err ? ORC_EINVAL : ORC_OK;
}

/* One row of an MXFP4 matrix decoded to fp32 (exact: E2M1 times a power of
 * two fits in fp32). */
static void mx_row_f32(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t r, float *out) {
  for (int64_t c = 0; c < K; ++c) out[c] = (float)mx_elem(codes, scales, K, r, c);
}

int orc_expert_ffn_f32(const float *x, int32_t nrows, const uint8_t *expert, int32_t d, int32_t f, float *y) {
  int64_t off[7];
  if (nrows < 0 || orc_expert_layout(d, f, off)) return ORC_EINVAL;
  if (nrows == 0) return ORC_OK;
  const uint8_t *gc = expert + off[0], *gs = expert + off[1];
  const uint8_t *uc = expert + off[2], *us = expert + off[3];
  const uint8_t *dc = expert + off[4], *ds = expert + off[5];
  float *h = (float *)malloc(sizeof(float) * (size_t)f * (size_t)nrows);
  if (!h) return ORC_EINVAL;
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t i = 0; i < f; ++i) {
    float *wg = (float *)malloc(sizeof(float) * (size_t)d * 2);
    if (!wg) { err |= 1; continue; }
    float *wu = wg + d;
    mx_row_f32(gc, gs, d, i, wg);
    mx_row_f32(uc, us, d, i, wu);
    for (int64_t n = 0; n < nrows; ++n) {
      float g = blocked_dot_f32(wg, x + n * d, d);
      float u = blocked_dot_f32(wu, x + n * d, d);
      float sg = g / (1.0f + expf(-g));
      h[n * f + i] = sg * u;
    }
    free(wg);
  }
  if (err) { free(h); return ORC_EINVAL; }
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t r = 0; r < d; ++r) {
    float *wd = (float *)malloc(sizeof(float) * (size_t)f);
    if (!wd) { err |= 1; continue; }
    mx_row_f32(dc, ds, f, r, wd);
    for (int64_t n = 0; n < nrows; ++n) y[n * d + r] = blocked_dot_f32(wd, h + n * f, f);
    free(wd);
  }
  free(h);
  return err ? ORC_EINVAL : ORC_OK;
}

/* Combine in fp32, one term after another in slot order: routed slots as
 * w * y (product rounded, then the add), shared slots added as they are. */
int orc_combine_f32(const float *y_slots, const float *w, int32_t M, int32_t k, int32_t S, int32_t d, float *out) {
  if (M < 0 || k < 1 || S < 0 || d <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * d; ++i) {
    int64_t m = i / d, r = i % d;
    float s = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      float t = w[m * k + j] * y_slots[(m * (k + S) + j) * d + r];
      s = s + t;
    }
    for (int64_t j = 0; j < S; ++j) s = s + y_slots[(m * (k + S) + k + j) * d + r];
    out[i] = s;
  }
  return ORC_OK;
}

/* Q8_0 in fp32: per 32-block b the sum of q[n,c] * X[m,c] over the block in
 * order, times the block's scale, the blocks added in ascending order. */
int orc_q8_0_matmul_f32(const float *X, int32_t M, int32_t K, const int8_t *wq, const uint16_t *ws, int32_t N,
                        float *Y) {
  if (M < 0 || K <= 0 || K % 32 || N <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * N; ++i) {
    int64_t m = i / N, n = i % N;
    float s = 0.0f;
    for (int64_t b = 0; b < K / 32; ++b) {
      float p = 0.0f;
      for (int64_t c = 32 * b; c < 32 * b + 32; ++c) {
        float t = (float)wq[n * K + c] * X[m * K + c];
        p = p + t;
      }
      float sb = (float)orc_fp16(ws[n * (K / 32) + b]);
      float t = sb * p;
      s = s + t;
    }
    Y[i] = s;
  }
  return ORC_OK;
}
