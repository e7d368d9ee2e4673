// Per-device state of the library.  Its one piece of device memory of its
// own: a fixed scratch array that stands in for the caller's backward
// workspace in fa_bwd_noalloc, for callers that cannot allocate (graph
// capture, serving loops that forbid allocation).  Each GPU holds its own copy for the life
// of the process.  Host code never passes `scratch` itself to a kernel (on
// the host it names a stand-in, not device memory): it takes the device
// address from hipGetSymbolAddress, looked up once per device with that
// device current, and passes that.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_launch.h"

namespace miattn {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Compute units of the current device, for the grid of persistent kernels.
hipError_t device_cu_count(int* n) {
  static std::mutex mu;
  static int cached[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] <= 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (v <= 0) return hipErrorInvalidValue;
    cached[dev] = v;
  }
  *n = cached[dev];
  return hipSuccess;
}

}  // namespace miattn
