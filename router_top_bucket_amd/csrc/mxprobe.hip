// One gfx950 MX-scaled matrix-core instruction, v_mfma_scale_f32_16x16x128_f8f6f4,
// with FP4 (E2M1) A and FP8 (E4M3) B operands and E8M0 block scales on both:
// the building block a prefill FFN would use to take MXFP4 weights without
// decoding them to bf16 ("Run Kimi 3.1 locally on one GPU", section "What is
// established—and what remains open": expert GEMM choices are among the
// arithmetic paths that can change near-tie tokens).  The library's
// FFN kernels do not use it: its sum of 128 products is not exact for
// activations that span many binades, which the GPU test of this entry point
// measures.  One wave computes D = A_s x B_s for one 16 x 16 x 128 tile.
//
// Operand layout in registers (lane l = r + 16 g, r = l % 16, g = l / 16):
//  - A: lane (r, g) holds row r, K [32 g, 32 g + 32) as 16 bytes of FP4
//    codes (element 2i in the low nibble of byte i);
//  - B: lane (r, g) holds column r, K [16 g, 16 g + 16) in bytes 0-15 and
//    K [64 + 16 g, 64 + 16 g + 16) in bytes 16-31, one FP8 code per byte;
//  - scales: lane (r, g) holds the E8M0 scale of row (A) or column (B) r for
//    the 32-element K block g, in byte 0 of its scale register;
//  - D: lane (r, g) holds D[4 g + t][r], t = 0..3, as the 16 x 16 MFMAs.
#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "common.h"

namespace moe {

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

constexpr int kMxFp8 = 0;  // operand format code of E4M3
constexpr int kMxFp4 = 4;  // operand format code of E2M1

__global__ __launch_bounds__(64) void mx_mfma_probe_kernel(const uint8_t *__restrict__ a_codes,
                                                           const uint8_t *__restrict__ a_scales,
                                                           const uint8_t *__restrict__ b_codes,
                                                           const uint8_t *__restrict__ b_scales,
                                                           float *__restrict__ d) {
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const u32x4 av = *(const u32x4 *)(a_codes + r * 64 + 16 * g);
  const u32x4 b0 = *(const u32x4 *)(b_codes + r * 128 + 16 * g);
  const u32x4 b1 = *(const u32x4 *)(b_codes + r * 128 + 64 + 16 * g);
  v8i32 a, b;
  for (int i = 0; i < 4; ++i) {
    a[i] = (int)av[i];
    a[4 + i] = 0;  // an FP4 operand occupies the first four registers
    b[i] = (int)b0[i];
    b[4 + i] = (int)b1[i];
  }
  const int sa = a_scales[r * 4 + g], sb = b_scales[r * 4 + g];
  const v4f32 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f32{0.f, 0.f, 0.f, 0.f}, kMxFp4, kMxFp8,
                                                                     0, sa, 0, sb);
  for (int t = 0; t < 4; ++t) d[(4 * g + t) * 16 + r] = acc[t];
}

}  // namespace moe

extern "C" int moe_mx_mfma_probe(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                                 const uint8_t *b_scales, float *d, void *stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !d) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(a_codes) % 16 || reinterpret_cast<uintptr_t>(b_codes) % 16) return MOE_EINVAL;
  hipLaunchKernelGGL(moe::mx_mfma_probe_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), a_codes,
                     a_scales, b_codes, b_scales, d);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
