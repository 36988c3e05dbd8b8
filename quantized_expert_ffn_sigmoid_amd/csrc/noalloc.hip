// noalloc.hip -- the device-resident workspace of moe_layer_forward_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid hipMalloc) run the layer on a workspace that the
// library carries as a file-scope device array: one copy per GPU, at its own
// address on each GPU, held until the process ends.  The array's name is a
// host-side stand-in in host code; the kernels receive the device address
// that hipGetSymbolAddress returns for the device the work runs on, looked up
// once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  // the device the stream's work runs on (the null stream: the current one)
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev, cur]() {
    // the lookup runs with that device current
    hipError_t r = dev == cur ? hipSuccess : hipSetDevice(dev);
    void* p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_err[dev] = r;
    g_ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
