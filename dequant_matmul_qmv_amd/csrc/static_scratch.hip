// Fixed device scratch for mxq_qmm_noalloc: the f32 partial results of split
// or chunked K live in a file-scope device array instead of allocated memory.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from the time the code object is loaded until the process ends.
// In host code `scratch` names a host-side stand-in, not a device address, so
// the address is looked up once per device (with that device current) and
// kept; kernels only ever receive that looked-up pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxq_internal.h"

namespace mxq {

static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mxq
