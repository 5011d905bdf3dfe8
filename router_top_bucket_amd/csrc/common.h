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

// Split a finite fp32 value into two bf16 parts: hi is v to the nearest bf16
// and lo the remainder (an exact fp32 difference) to the nearest bf16, so
// |v - hi - lo| <= 2^-18 |v|.
__device__ __forceinline__ void split2_bf16(float v, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// ---- buffer loads: a 32-bit byte offset into a resource of `bytes` bytes.
// An offset past the end reads as zero and never faults, so masked lanes and
// ragged tails need no branch around the load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Every resource here is smaller than 2^30 bytes.  An invalid lane's base
// offset is kOOB and a dead step adds kDead, so any sum involving either is
// at least 2^30 (past the end) and at most ~3.3 * 2^30 (no 32-bit wrap).
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kDead = 0x40000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same load marked non-temporal (nt): for a stream read once, so that
// its lines leave the caches first and data that is re-read stays.
__device__ __forceinline__ u32x4 buf_load16_stream(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t sel_off(bool ok, uint32_t off) { return ok ? off : kOOB; }

// s_waitcnt operand (gfx9 encoding) that waits for every vector-memory load
// of the wave and nothing else: vmcnt 0, expcnt 7, lgkmcnt 15.
constexpr int kWaitVmcnt0 = 0x0F70;

// Workgroup barrier for handing LDS data between waves: waits for this wave's
// LDS operations only.  __syncthreads() is a full workgroup fence and would
// also wait for every global load the wave has in flight, draining any
// prefetch ring at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- direct loads into LDS (gfx950 LDS DMA).  Lane l of one instruction
// writes its 16 bytes to lds_base + 16 l (lds_base is wave-uniform), so one
// instruction fills 1 KB of LDS in lane order; which global bytes land where
// is chosen by each lane's offset.  The load is counted by vmcnt like any
// other and its data is in LDS once this wave's vmcnt has passed it.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint32_t off, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, off, 0, 0, 0);
}
// Wait until at most N vector-memory loads of this wave are in flight
// (s_waitcnt vmcnt(N), gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Barrier for LDS filled by LDS DMA: this wave's LDS reads and writes are
// done, then s_barrier.  No fence: a workgroup fence makes the compiler wait
// for every load in flight (LDS DMA included), which would drain the ring;
// the caller waits for the DMA loads it needs with wait_vmcnt.  The memory
// clobber keeps every memory access on its side of the barrier.
__device__ __forceinline__ void lds_dma_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- wave reductions without LDS: DPP inside each 16-lane row, then the four
// row results read as scalars and combined in row order.  Every lane of a
// row ends with bit-identical values (each step combines a lane with a fixed
// partner; a + b == b + a and max is symmetric), so the result is uniform and
// independent of which lane asks.
#define MOE_DPP_QUAD_1032 0xB1  // quad_perm [1,0,3,2]
#define MOE_DPP_QUAD_2301 0x4E  // quad_perm [2,3,0,1]
#define MOE_DPP_ROW_HALF_MIRROR 0x141
#define MOE_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum over the 64 lanes: ((row0 + row1) + row2) + row3 of fixed-tree row sums.
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f32<MOE_DPP_QUAD_1032>(v);
  v = v + dpp_f32<MOE_DPP_QUAD_2301>(v);
  v = v + dpp_f32<MOE_DPP_ROW_HALF_MIRROR>(v);
  v = v + dpp_f32<MOE_DPP_ROW_MIRROR>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  return max_u64(v, ((uint64_t)hi << 32) | lo);
}

// Maximum over the 64 lanes (uniform result).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<MOE_DPP_QUAD_1032>(v);
  v = dpp_max_u64<MOE_DPP_QUAD_2301>(v);
  v = dpp_max_u64<MOE_DPP_ROW_HALF_MIRROR>(v);
  v = dpp_max_u64<MOE_DPP_ROW_MIRROR>(v);
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, row * 16);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), row * 16);
    r = max_u64(r, ((uint64_t)hi << 32) | lo);
  }
  return r;
}

}  // namespace moe
