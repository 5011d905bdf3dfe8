// Device-side building blocks shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

namespace moe {

constexpr int kWave = 64;

// E8M0 scale byte -> fp32 2^(b-127).  b = 0 is the subnormal 2^-127; b = 255
// is NaN by the format and outside the supported input range.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble of byte 0) times a
// power-of-two scale, as eight bf16.  Exact: an E2M1 value has 2 significant
// bits, so value*2^k is representable in bf16 for every scale in range.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// D += A * B over K = 32 for a 16x16 tile.  Lane l supplies A[l%16][8*(l/16)+i]
// and B[8*(l/16)+i][l%16] (i = 0..7) and holds D[4*(l/16)+i][l%16] (i = 0..3).
// Each D element is a function of its own A row and B column only.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split a finite fp32 value into three bf16 parts with v == hi + mid + lo
// exactly (each part takes the next 8 significant bits of the remainder; the
// remainders are exact fp32 differences).
__device__ __forceinline__ void split3_bf16(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  hi = f32_to_bf16_bits(v);
  float r1 = v - bf16_bits_to_f32(hi);
  mid = f32_to_bf16_bits(r1);
  float r2 = r1 - bf16_bits_to_f32(mid);
  lo = f32_to_bf16_bits(r2);
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace moe
