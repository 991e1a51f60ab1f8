// The draft step on a fixed scratch buffer of the library's own, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the workspace mtp_draft_step takes
// from its caller lives here instead, in a file-scope device array that every
// GPU the library runs on holds until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device address:
// its address on each device comes from hipGetSymbolAddress, taken once per
// device (with that device current) at the first call there, and only that
// address is passed to kernels. The first call on a device also clears the
// lm_head's completion counter and running maxima with a fill kernel (no
// hipMemsetAsync, so a captured first call records no memset node); every call
// leaves them at zero again. All calls on one GPU share that GPU's array:
// calls that overlap in time (different streams) race.
#include <mutex>

#include "mtp_kernels.h"

namespace mtp {

namespace {

static __device__ __align__(256) uint8_t scratch[kStepScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];

// Zeroes n 32-bit words at p (one thread per word).
__global__ void scratch_clear_kernel(uint32_t *p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

// This device's address of the array; at the first call on the device, the
// counters are cleared on `s` before anything else uses them.
hipError_t scratch_on_device(hipStream_t s, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    constexpr int kWords = (int)(kLmheadKmaxOffset + 8 * 8) / 4;  // ticket and running maxima
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(64), 0, s, static_cast<uint32_t *>(ptr), kWords);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_step_scratch(const StepLaunch &a, hipStream_t s) {
  if (step_ws_bytes(a.c.b, a.c.h) > kStepScratchBytes) return hipErrorInvalidValue;
  void *ptr = nullptr;
  const hipError_t e = scratch_on_device(s, &ptr);
  if (e != hipSuccess) return e;
  StepLaunch b = a;
  b.ws = ptr;
  return launch_step(b, s);
}

}  // namespace mtp
