// Read probe: how fast this GPU streams a buffer of a given size with the
// load form the decode kernel uses (16-byte non-temporal loads, 1 KiB of
// contiguous data per wave instruction, four loads in flight per lane, two
// 256-thread workgroups per compute unit).  A measurement aid: the fused
// kernels' bandwidth at a given size is judged against this curve, since a
// small read cannot reach the HBM peak however it is done.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {
constexpr uint32_t kNever = 0x9E3779B9u;  // an XOR of the data equal to this writes it out
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u4* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4 a = __builtin_nontemporal_load(p + i);
    const u4 b = __builtin_nontemporal_load(p + i + stride);
    const u4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // the data decides whether anything is written, so no load can be dropped
  if (acc == kNever) out[0] = acc;
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream,
                             const DeviceInfo& dev) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 4 * 256 - 1) / (4 * 256);
  const int64_t cap = static_cast<int64_t>(dev.num_cu) * 2;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const u4*>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace mxq
