// Library-owned scratch for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): a file-scope device array that stands in for the caller
// workspace of q1_qmm.  Each GPU the library runs on holds its own copy until
// the process ends.  Every call on one GPU shares that GPU's array, so calls
// that overlap on one GPU race; calls ordered on one stream do not.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "q1_internal.h"

namespace q1 {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Clears the arrival counters at the start of the array (a kernel, not a
// memset node, so that a captured graph replays it correctly).
__global__ void q1_clear_counters(uint32_t* p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x)) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device (nullptr: not set up)

}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    // set-up on this device (current): the host-side name `scratch` is not a
    // device address; only the address returned here is passed to kernels
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // the counters must start at zero; every call leaves them zero again
    hipLaunchKernelGGL(q1_clear_counters, dim3(16), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       (int)(kCounterBytes / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace q1
