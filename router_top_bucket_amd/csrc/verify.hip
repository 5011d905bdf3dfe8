// Small kernels of the block-verification harness ("Run Kimi 3.1 locally on
// one GPU", section "A drafter that leaves the answer unchanged", and its run
// record).  The harness compares a multi-row verification block with one-row
// steps: block outputs must match bit for bit, a draft is accepted only while
// it equals the greedy choice, and every position's logits are FNV-1a
// hashed on both sides.  The lookups, adds, casts, argmax and hashes are exact;
// the RMS normalisation is fp32 in an order fixed by the row length.
#include "common.h"
#include "launch.h"

namespace moe {

// ---- rows of a Q8_0 matrix as fp32: X[m, c] = Wq[ids[m], c] * Ws[ids[m], c/32]
// (the product of an int8 and an fp16 is exact in fp32), Wq in row or tile
// order.  One thread per 4 consecutive c.  Ids outside [0, N) give a zero row.
__global__ void q8_0_rows_kernel(const int32_t *__restrict__ ids, int M, int K, const int8_t *__restrict__ wq,
                                 const uint16_t *__restrict__ ws, int N, float *__restrict__ X, int tiled) {
  const int K4 = K >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * K4) return;
  const int m = (int)(idx / K4), c = (int)(idx - (int64_t)m * K4) * 4;
  const int id = ids[m];
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
  if (id >= 0 && id < N) {
    // tile order (q8_0.hip): block c/32 of row id at ((id/16)*(K/32) + c/32)*512 + (id%16)*32
    const int64_t off = tiled ? (((int64_t)(id >> 4) * (K >> 5) + (c >> 5)) * 512 + (id & 15) * 32 + (c & 31))
                              : (int64_t)id * K + c;
    const uint32_t q = *(const uint32_t *)(wq + off);
    const float s = (float)__builtin_bit_cast(_Float16, ws[(int64_t)id * (K >> 5) + (c >> 5)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)(int8_t)(q >> (8 * i)) * s;
  }
  *(f32x4 *)(X + (int64_t)m * K + c) = v;
}

// ---- h += a (if a), then hb = bf16(h) rounded to nearest even (if hb)
__global__ void residual_bf16_kernel(float *__restrict__ h, const float *__restrict__ a, int64_t n,
                                     uint16_t *__restrict__ hb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = h[i];
  if (a) {
    v = v + a[i];
    h[i] = v;
  }
  if (hb) hb[i] = (uint16_t)f32_to_bf16_bits(v);
}

// ---- RMS normalisation per row without a gain vector:
// r = 1 / sqrt(sum_c h[c]^2 / d + eps), out[c] = h[c] * r, as fp32 and/or as
// bf16 bits (round to nearest even).  One workgroup per row.  Rows of up to
// RN_THREADS*4*RN_VEC elements with d % 4 == 0 stay in registers (float4 loads,
// all issued before the sum); others are read twice.  The sum: each thread
// adds its elements in ascending order, then a fixed DPP tree per wave and
// the waves in order; the order depends only on d, never on M.
constexpr int RN_THREADS = 256, RN_VEC = 8;
__global__ __launch_bounds__(RN_THREADS) void rmsnorm_kernel(const float *__restrict__ h, int d, float eps,
                                                             float *__restrict__ out, uint16_t *__restrict__ outb) {
  __shared__ float part[RN_THREADS / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float *row = h + (int64_t)m * d;
  const bool regs = (d & 3) == 0 && d <= RN_THREADS * 4 * RN_VEC;
  f32x4 v[RN_VEC];
  float s = 0.f;
  if (regs) {
#pragma unroll
    for (int j = 0; j < RN_VEC; ++j) {
      const int c = 4 * (tid + j * RN_THREADS);
      v[j] = c < d ? *(const f32x4 *)(row + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < RN_VEC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = __builtin_fmaf(v[j][i], v[j][i], s);
  } else {
    for (int i = tid; i < d; i += RN_THREADS) s = __builtin_fmaf(row[i], row[i], s);
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float r = 1.0f / __builtin_sqrtf(tot / (float)d + eps);
  if (regs) {
#pragma unroll
    for (int j = 0; j < RN_VEC; ++j) {
      const int c = 4 * (tid + j * RN_THREADS);
      if (c < d) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[j][i] * r;
        if (out) *(f32x4 *)(out + (int64_t)m * d + c) = o;
        if (outb) {
          const uint32_t b0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
          const uint32_t b1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
          *(uint2 *)(outb + (int64_t)m * d + c) = make_uint2(b0, b1);
        }
      }
    }
  } else {
    for (int i = tid; i < d; i += RN_THREADS) {
      const float o = row[i] * r;
      if (out) out[(int64_t)m * d + i] = o;
      if (outb) outb[(int64_t)m * d + i] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
}

// ---- per row: the index of the largest value (NaN below every number, the
// lowest index among equal values).  One 1024-thread workgroup per row; with
// N % 4 == 0 each thread takes float4 pieces AM_UNROLL at a time (all loads of
// a round issued before their compares), else single elements.  The (value,
// index) keys are then reduced over the wave and the workgroup; the key
// order is total, so the reduction order cannot change the answer.
constexpr int AM_THREADS = 1024, AM_UNROLL = 4;
__device__ __forceinline__ uint64_t am_key(float v, int i) {
  if (v != v) v = -INFINITY;
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __float_as_uint(v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)i;
}
__global__ __launch_bounds__(AM_THREADS) void argmax_rows_kernel(const float *__restrict__ X, int N,
                                                                 int32_t *__restrict__ idx) {
  __shared__ uint64_t part[AM_THREADS / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float *row = X + (int64_t)m * N;
  uint64_t best = 0;
  if ((N & 3) == 0) {
    const int n4 = N >> 2;
    for (int base = 0; base < n4; base += AM_THREADS * AM_UNROLL) {
      f32x4 v[AM_UNROLL];
#pragma unroll
      for (int u = 0; u < AM_UNROLL; ++u) {
        const int p = base + u * AM_THREADS + tid;
        v[u] = *(const f32x4 *)(row + 4 * (p < n4 ? p : n4 - 1));
      }
#pragma unroll
      for (int u = 0; u < AM_UNROLL; ++u) {
        const int p = base + u * AM_THREADS + tid;
        if (p < n4)
#pragma unroll
          for (int i = 0; i < 4; ++i) best = max_u64(best, am_key(v[u][i], 4 * p + i));
      }
    }
  } else {
    for (int i = tid; i < N; i += AM_THREADS) best = max_u64(best, am_key(row[i], i));
  }
  best = wave_max_u64(best);
  if ((tid & 63) == 0) part[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = part[0];
    for (int w = 1; w < AM_THREADS / 64; ++w) b = max_u64(b, part[w]);
    idx[m] = (int32_t)~(uint32_t)b;
  }
}

// ---- per row: 64-bit FNV-1a over the row's bytes in memory order (fp32,
// little endian).  FNV-1a is a sequential recurrence, so one thread walks one
// row: h = (h ^ byte) * 0x100000001b3 from h = 0xcbf29ce484222325.
__global__ void fnv1a_rows_kernel(const float *__restrict__ X, int M, int N, uint64_t *__restrict__ hash) {
  const int m = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (m >= M) return;
  const uint32_t *row = (const uint32_t *)(X + (int64_t)m * N);
  uint64_t h = 0xcbf29ce484222325ull;
  for (int i = 0; i < N; ++i) {
    const uint32_t w = row[i];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h ^= (w >> (8 * b)) & 0xFFu;
      h *= 0x100000001b3ull;
    }
  }
  hash[m] = h;
}

int q8_0_rows_launch(const int32_t *ids, int M, int K, const int8_t *wq, const uint16_t *ws, int N, float *X,
                     int tiled, hipStream_t stream) {
  const int64_t n = (int64_t)M * (K / 4);
  hipLaunchKernelGGL(q8_0_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ids, M, K, wq, ws, N,
                     X, tiled);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int residual_bf16_launch(float *h, const float *a, int64_t n, uint16_t *hb, hipStream_t stream) {
  hipLaunchKernelGGL(residual_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h, a, n, hb);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int rmsnorm_launch(const float *h, int M, int d, float eps, float *out, uint16_t *outb, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(RN_THREADS), 0, stream, h, d, eps, out, outb);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int argmax_rows_launch(const float *X, int M, int N, int32_t *idx, hipStream_t stream) {
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(M), dim3(AM_THREADS), 0, stream, X, N, idx);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fnv1a_rows_launch(const float *X, int M, int N, uint64_t *hash, hipStream_t stream) {
  hipLaunchKernelGGL(fnv1a_rows_kernel, dim3((M + 63) / 64), dim3(64), 0, stream, X, M, N, hash);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace moe
