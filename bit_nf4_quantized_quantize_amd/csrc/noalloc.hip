// The forward of the linear layer for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc): qlora_linear_fwd with its workspace taken from a fixed
// array of the library's own device memory instead of a caller buffer.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy from the time the code object is loaded there until the
// process ends.  In host code its name is only a host-side stand-in, so the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; only that address
// ever reaches a kernel.  Nothing here allocates.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "launch.h"
#include "qlora_nf4.h"

namespace {

constexpr int64_t kScratchBytes = (int64_t)96 << 20;  // the forward's largest workspace at the workload shapes is 72 MiB
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's `scratch` (looked up on the first call on
// the device), or the failure status.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "qlora_linear_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return qlora::record_failure(QLORA_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return qlora::record_failure(QLORA_ERR_INVALID_ARG, "qlora_linear_fwd_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof(msg), "qlora_linear_fwd_noalloc: hipGetSymbolAddress(scratch): %s",
               hipGetErrorString(e));
      return qlora::record_failure(QLORA_ERR_HIP, msg);
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const void* X, int64_t M, const qlora_nf4_t* W, const void* A, const void* B,
                                        int32_t r, float s, void* Y, void* XA, void* stream) {
  // shape errors are reported by the plain entry point's own validation
  int64_t need = 0;
  const bool sized = W && qlora_linear_workspace(M, W->rows, W->cols, r, &need, nullptr) == QLORA_OK;
  if (sized && need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "qlora_linear_fwd_noalloc: this call needs %lld bytes of scratch, above the fixed capacity of %lld "
             "bytes (use qlora_linear_fwd with a workspace)",
             (long long)need, (long long)kScratchBytes);
    return qlora::record_failure(QLORA_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  void* ws = nullptr;
  if (sized && M > 0) {
    const int st = scratch_of_current_device(&ws);
    if (st) return st;
  }
  return qlora_linear_fwd(X, M, W, A, B, r, s, Y, XA, ws, ws ? kScratchBytes : 0, stream);
}
