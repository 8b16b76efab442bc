// Device scratch of mamba_scan_fwd_noalloc: the prefill's chunk summaries
// and state copies (the workspace mamba_scan_fwd takes from its caller) kept
// in a fixed array of the library, for callers that cannot allocate device
// memory. Every device the library runs on holds its own copy of the array
// until the process ends; all calls on one device share it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mamba_scan.h"
#include "scan_internal.h"

namespace mscan {

constexpr size_t kNoallocScratchBytes = MAMBA_SCAN_NOALLOC_SCRATCH_BYTES;  // 8 MiB

static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

// The device address of `scratch` on device `dev`, which must be the current
// device: looked up with hipGetSymbolAddress on the first call for that
// device, then reused. In host code the name `scratch` is only a host-side
// stand-in, so kernels and copies always get this address instead.
hipError_t noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mscan
