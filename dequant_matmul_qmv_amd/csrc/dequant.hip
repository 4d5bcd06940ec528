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
// W (rows of K codes, K / (32 / bits) words each), the scales and biases
// ([N, K / g], K a multiple of g) and out ([N, K]) are all contiguous, so the
// operation is elementwise over the N * K codes taken in order: code c sits in
// word c / (32 / bits) at field c % (32 / bits), and its scale and bias at
// index c / g.  Thread unit t produces the outputs of codes [V t, V t + V),
// one 16-byte store (V = 4 for f32 output, 8 for f16 / bf16), so each store
// instruction of a wave writes 1 KiB of contiguous output; V divides every
// group size, so a unit never straddles a group.  Each thread runs four units
// per loop trip, their loads issued first.  The output is written once and
// not read back here, so the stores are non-temporal (measured on lm_head,
// 4-bit to f32: 303 -> 228 us; 8-bit to f32 with non-temporal loads as well:
// 293 -> 259 us).
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

template <int BITS, bool SB_BF16, int OUT>  // OUT: 0 f16, 1 bf16, 2 f32
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ W,
                                                      const uint16_t* __restrict__ S,
                                                      const uint16_t* __restrict__ B,
                                                      void* __restrict__ out, int64_t nunits, int glog2) {
  constexpr int V = OUT == 2 ? 4 : 8;             // codes per unit (one 16-byte store)
  constexpr int CPW = 32 / BITS;                  // codes per word
  constexpr int NW = (V * BITS + 31) / 32;        // words a unit reads (1, or 2 for 8-bit codes to f16)
  constexpr int UNROLL = 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t0 < nunits;
       t0 += UNROLL * stride) {
    uint32_t wv[UNROLL][NW];
    uint16_t sv[UNROLL], bv[UNROLL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int64_t t = min(t0 + j * stride, nunits - 1);  // loads clamped; stores guarded below
      const int64_t c0 = t * V;
      const int64_t w0 = c0 / CPW;
      if constexpr (NW == 2) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(W + w0));
        wv[j][0] = v.x;
        wv[j][1] = v.y;
      } else {
        // 8-bit codes: each word is read by one lane, once, so non-temporal;
        // 4-bit codes to f32 share a word between two lanes, and plain loads
        // measured faster there
        wv[j][0] = BITS == 8 ? __builtin_nontemporal_load(W + w0) : W[w0];
      }
      sv[j] = S[c0 >> glog2];
      bv[j] = B[c0 >> glog2];
    }
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int64_t t = t0 + j * stride;
      if (t >= nunits) break;
      const int64_t c0 = t * V;
      const float s = sb_to_f32<SB_BF16>(sv[j]);
      const float b = sb_to_f32<SB_BF16>(bv[j]);
      // first field of this unit in its (first) word: 4-bit codes to f32 take
      // half a word, the other layouts whole words
      const int f0 = static_cast<int>(c0 % CPW);
      float v[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int f = f0 + i;
        const uint32_t word = wv[j][NW == 2 ? i / CPW : 0];
        const float q = static_cast<float>((word >> (BITS * (NW == 2 ? f % CPW : f))) & ((1u << BITS) - 1u));
        v[i] = __fadd_rn(__fmul_rn(q, s), b);
      }
      if constexpr (OUT == 2) {
        __builtin_nontemporal_store(
            u4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])},
            reinterpret_cast<u4*>(static_cast<float*>(out) + c0));
      } else {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = (OUT == 0) ? f32_to_f16_bits(v[2 * i]) : f32_to_bf16_bits(v[2 * i]);
          const uint32_t hi = (OUT == 0) ? f32_to_f16_bits(v[2 * i + 1]) : f32_to_bf16_bits(v[2 * i + 1]);
          p[i] = lo | (hi << 16);
        }
        __builtin_nontemporal_store(u4{p[0], p[1], p[2], p[3]}, reinterpret_cast<u4*>(static_cast<uint16_t*>(out) + c0));
      }
    }
  }
}

template <int BITS, bool SB_BF16>
static hipError_t launch_dq(const DequantArgs& a, const DeviceInfo& dev) {
  const int64_t V = a.out_dtype == 2 ? 4 : 8;  // f32 output: 4 codes per 16-byte store, else 8
  const int64_t nunits = a.N * a.K / V;
  int64_t blocks = (nunits + 4 * 256 - 1) / (4 * 256);
  const int64_t cap = static_cast<int64_t>(dev.num_cu) * 16;
  if (blocks > cap) blocks = cap;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (a.out_dtype) {
    case 0: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 0>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, a.glog2); break;
    case 1: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 1>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, a.glog2); break;
    default: hipLaunchKernelGGL((dequant_kernel<BITS, SB_BF16, 2>), grid, block, 0, a.stream, a.w, a.s, a.b, a.out, nunits, a.glog2); break;
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
