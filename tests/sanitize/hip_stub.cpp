// Host-only stand-in for the few HIP runtime calls libmxq's C-ABI layer
// makes, so that api.cpp and workspace.cpp can be built and run under
// AddressSanitizer / UndefinedBehaviorSanitizer on a machine without a GPU.
// Two fake devices (256 compute units, 160 KiB of LDS); hipMalloc / hipFree
// are malloc / free (so the sanitizer sees every workspace buffer), with a
// switch that makes allocations fail.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>

namespace {
thread_local int t_device = 0;
std::atomic<int> g_fail_malloc{0};
std::atomic<long> g_live{0};
}  // namespace

extern "C" void stub_fail_malloc(int on) { g_fail_malloc = on; }
extern "C" long stub_live_allocations(void) { return g_live.load(); }

hipError_t hipGetDevice(int* d) {
  *d = t_device;
  return hipSuccess;
}

hipError_t hipSetDevice(int d) {
  if (d < 0 || d > 1) return hipErrorInvalidDevice;
  t_device = d;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int d) {
  if (d < 0 || d > 1) return hipErrorInvalidDevice;
  switch (attr) {
    case hipDeviceAttributeMultiprocessorCount: *v = 256; return hipSuccess;
    case hipDeviceAttributeMaxSharedMemoryPerBlock: *v = 160 * 1024; return hipSuccess;
    case hipDeviceAttributeMaxSharedMemoryPerMultiprocessor: *v = 160 * 1024; return hipSuccess;
    default: *v = 0; return hipSuccess;
  }
}

hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipSuccess; }
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) {
  *n = 2;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorName(hipError_t) { return "hipErrorStub"; }
const char* hipGetErrorString(hipError_t) { return "stub error"; }

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
  *s = hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipMalloc(void** p, size_t bytes) {
  if (g_fail_malloc) {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  *p = std::malloc(bytes ? bytes : 1);
  if (*p == nullptr) return hipErrorOutOfMemory;
  ++g_live;
  return hipSuccess;
}

hipError_t hipFree(void* p) {
  if (p != nullptr) {
    --g_live;
    std::free(p);
  }
  return hipSuccess;
}
