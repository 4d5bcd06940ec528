// Standalone dequantization: out[n, k] = q * s + b, bit-exact.
//
// mlxcel #574 "What is already in-tree": the reconstruction (bit-unpack, then
// q*scale + bias) must be bit-identical to a host dequant.  q*s is exact in f32
// (a code has at most 8 significant bits, an f16 scale 11, a bf16 scale 8), so
// the f32 multiply followed by the f32 add rounds exactly once, the same as a
// fused multiply-add: the value is RN_f32(q*s + b) whichever the compiler picks.
// f16 / bf16 outputs round that f32 value to nearest even.  This path writes the
// weight out by design (it is the bit-exact anchor, not the fused path).
//
// One thread handles one 16-byte segment of a row (32 4-bit or 16 8-bit codes,
// always inside one group) and writes its outputs as 16-byte stores.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

template <int BITS, bool SB_BF16, int OUT>  // OUT: 0 f16, 1 bf16, 2 f32
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ W,
                                                      const uint16_t* __restrict__ S,
                                                      const uint16_t* __restrict__ B,
                                                      void* __restrict__ out, int64_t nunits,
                                                      int nseg, int K, int glog2) {
  constexpr int CODES = 128 / BITS;
  constexpr int PER = 32 / BITS;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < nunits; u += stride) {
    const int64_t row = u / nseg;
    const int seg = static_cast<int>(u - row * nseg);
    const int G = K >> glog2;
    const u4 wv = *reinterpret_cast<const u4*>(W + row * (K / PER) + seg * 4);
    const int grp = (seg * CODES) >> glog2;
    const float s = sb_to_f32<SB_BF16>(S[row * G + grp]);
    const float b = sb_to_f32<SB_BF16>(B[row * G + grp]);
    const uint32_t wr[4] = {wv.x, wv.y, wv.z, wv.w};
    float v[CODES];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int c = 0; c < PER; ++c) {
        const float q = static_cast<float>((wr[i] >> (BITS * c)) & ((1u << BITS) - 1u));
        v[i * PER + c] = __fadd_rn(__fmul_rn(q, s), b);
      }
    }
    const int64_t base = row * K + static_cast<int64_t>(seg) * CODES;
    if constexpr (OUT == 2) {
      u4* o = reinterpret_cast<u4*>(static_cast<float*>(out) + base);
#pragma unroll
      for (int c = 0; c < CODES / 4; ++c)
        o[c] = u4{__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]),
                  __float_as_uint(v[4 * c + 2]), __float_as_uint(v[4 * c + 3])};
    } else {
      u4* o = reinterpret_cast<u4*>(static_cast<uint16_t*>(out) + base);
#pragma unroll
      for (int c = 0; c < CODES / 8; ++c) {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = v[8 * c + 2 * i], a1 = v[8 * c + 2 * i + 1];
          const uint32_t lo = (OUT == 0) ? f32_to_f16_bits(a0) : f32_to_bf16_bits(a0);
          const uint32_t hi = (OUT == 0) ? f32_to_f16_bits(a1) : f32_to_bf16_bits(a1);
          p[i] = lo | (hi << 16);
        }
        o[c] = u4{p[0], p[1], p[2], p[3]};
      }
    }
  }
}

template <int BITS, bool SB_BF16>
static hipError_t launch_dq(const DequantArgs& a, const DeviceInfo& dev) {
  const int nseg = static_cast<int>(a.K * BITS / 128);
  const int64_t nunits = a.N * nseg;
  int64_t blocks = (nunits + 255) / 256;
  const int64_t cap = static_cast<int64_t>(dev.num_cu) * 16;
  if (blocks > cap) blocks = cap;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int K = static_cast<int>(a.K);
  switch (a.out_dtype) {
    case 0: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 0>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, nseg, K, a.glog2); break;
    case 1: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 1>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, nseg, K, a.glog2); break;
    default: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 2>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, nseg, K, a.glog2); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, const DeviceInfo& dev) {
  if (a.bits == 4) return a.sb_bf16 ? launch_dq<4, true>(a, dev) : launch_dq<4, false>(a, dev);
  return a.sb_bf16 ? launch_dq<8, true>(a, dev) : launch_dq<8, false>(a, dev);
}

__global__ void zero_fill_kernel(uint16_t* __restrict__ y, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
    y[i] = 0;
}

__global__ void fill_rows_kernel(uint16_t* __restrict__ y, const uint16_t* __restrict__ ob, int64_t M, int64_t N) {
  const int64_t count = M * N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
    y[i] = ob[i % N];
}

hipError_t launch_fill_rows(uint16_t* y, const uint16_t* ob, int64_t M, int64_t N, hipStream_t stream) {
  if (!ob) return launch_zero_fill(y, M * N, stream);
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, y, ob, M, N);
  return hipGetLastError();
}

hipError_t launch_zero_fill(uint16_t* y, int64_t count, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, y, count);
  return hipGetLastError();
}

}  // namespace mxq
