// noalloc.hip - the library-held scratch of the allocation-free linear
// (paro_w4a16_linear_noalloc in include/paro.h).
//
// The workspace of the linear (split-K counters and partial sums, the rotated
// activations, the prefill path's dense rotation) lives here in a file-scope
// device array, one copy per GPU for the life of the process, so that callers
// that cannot allocate (graph capture, tight serving loops) still run the
// linear.  Host code never uses the array's name as an address: on the first
// call on a device, with that device current, hipGetSymbolAddress gives the
// device's own address of its copy, which is kept per device and passed to
// the kernels like any caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[paro::kNoallocScratchBytes];

namespace paro {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void *ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_mutex;

__global__ void __launch_bounds__(256) zero_fill_kernel(uint4 *__restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t st, size_t zero_bytes, void **ptr) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch &d = g_scratch[dev];
  if (!d.ptr) {
    // first use on this device: no graph capture may be under way, since the
    // clearing below must run before any later call, captured or not
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(st, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
      // the split-K counters must start at zero (every call leaves them zero)
      const size_t n16 = zero_bytes / 16;
      const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
      if (n16) hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, st, (uint4 *)p, n16);
      e = hipGetLastError();
    }
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    d.ptr = p;
  }
  *ptr = d.ptr;
  return hipSuccess;
}

}  // namespace paro
