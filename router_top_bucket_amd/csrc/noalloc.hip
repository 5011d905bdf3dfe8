// moe_layer_mxfp4_noalloc: the layer call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Its kernels are moe_layer_mxfp4's; their scratch
// (the hidden activations h and, above 16 rows, the group plan) lives in a
// file-scope device array of fixed size instead of a caller's workspace.
//
// The array is a device symbol: in host code its name stands for a host-side
// shadow, not for device memory, so host code never passes it to a kernel or
// a copy.  Each device gets the array's device address once, with that device
// current, from hipGetSymbolAddress; every launch then uses that address.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/moe.h"
#include "checks.h"
#include "launch.h"

namespace {

// 8 MiB: a Kimi-shaped layer (d = 7168, f = 1536, k = 16, S = 2) needs
// 1.77 MB at 16 rows and fits up to 75 rows.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The array's address on the device that runs `stream` (its device, or the
// current device for the null stream), looked up once per device with that
// device current.  Null if the device cannot be determined or the lookup
// fails.
void *device_scratch(hipStream_t stream) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return nullptr;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
  void *addr = nullptr;
  const hipError_t rc = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (dev != cur) (void)hipSetDevice(cur);
  if (rc != hipSuccess || !addr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_layer_mxfp4_noalloc(const void *x, moe_dtype x_dtype, const float *w_router, float *logits, int32_t M,
                            int32_t k, const moe_experts *W, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                            int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error, float *y_slots,
                            float *out, void *stream) {
  // every argument check of moe_layer_mxfp4 except the workspace size (the
  // workspace is the scratch array; a stand-in pointer passes the checks and
  // nothing is read through it), then the size against the array's
  static const uint8_t stand_in[256] __attribute__((aligned(256))) = {};
  const int rc = moe_layer_check(x, x_dtype, w_router, logits, M, k, W, topk_ids, topk_w, offsets, perm, active,
                                 n_active, dev_error, y_slots, out, stand_in, SIZE_MAX);
  if (rc != MOE_OK) return rc;
  if (M == 0) return MOE_OK;
  if (moe_workspace_bytes(M, k, W) > kScratchBytes) return MOE_ESCRATCH;
  void *ws = device_scratch(reinterpret_cast<hipStream_t>(stream));
  if (!ws) return MOE_EHIP;
  return moe_layer_enqueue(x, x_dtype, w_router, logits, M, k, W, topk_ids, topk_w, offsets, perm, active, n_active,
                           dev_error, y_slots, out, ws, stream);
}

}  // extern "C"
