// Device-side helpers shared by the gfx950 kernels of libmxq.
//
// Packed layout (mlxcel epic #570 "Context": a uint32 payload plus per-group
// f16 / bf16 scales and biases; mlxcel #574 "What is already in-tree":
// bit-unpack, then q*scale + bias).  Code i of a word sits in bits
// [bits*i, bits*i + bits), least significant field first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Pointers into the global address space: loads through them are global_load
// instructions even when the compiler cannot trace them to a kernel argument.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return reinterpret_cast<gptr<T>>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Exact widening of a stored scale / bias to f32.
template <bool BF16>
__device__ __forceinline__ float sb_to_f32(uint16_t u) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, u));
  }
}

// ---------------------------------------------------------------------------
// Exact f16 codes by exponent injection.  OR-ing a code c < 1024 into the
// mantissa of the f16 1024.0 (bits 0x6400) gives the f16 value 1024 + c, and
// subtracting 1024 afterwards is exact, so each half holds the integer code
// itself.  The helpers named _off leave a power-of-two offset in instead, for
// callers that remove it through the group's bias.  One v_and_or_b32 builds
// two codes at once; the pairs come out as (c0, c4), (c1, c5), (c2, c6),
// (c3, c7) for a 4-bit word and (c0, c2), (c1, c3) for an 8-bit word, and the
// decode kernel stages its activations in that same order, so each v_dot2
// multiplies matching (code, x) pairs.
// ---------------------------------------------------------------------------
constexpr uint32_t kMagic = 0x64006400u;

__device__ __forceinline__ h2 sub1024(uint32_t u) {
  const h2 k = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  return as_h2(u) - k;
}

// (a & mask) | c in one v_and_or_b32.  gfx9 VOP3 takes no literal constants
// and reads at most one SGPR, so the mask goes in an SGPR and c in a VGPR;
// left to itself the compiler splits this into v_and + v_or.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(c));
  return d;
}

// f16 pattern of 64 in both halves.  Mantissa bits 4..7 under this exponent
// weigh exactly 1, so a code placed there reads as 64 + c.
constexpr uint32_t kMagic64 = 0x54005400u;

// 4-bit word -> (64 + c0, 64 + c4), (64 + c1, 64 + c5), (64 + c2, 64 + c6),
// (64 + c3, 64 + c7) as f16 pairs, exact: every code is moved to bits 4..7 of
// its half (shifts by +4, 0, -4, -8) and injected under the exponent of 64
// (`magic` = kMagic64), 7 ops per word.  The offset is left in; callers remove
// 64 * sum(x) through the group's bias.
__device__ __forceinline__ void unpack_w4_off64(uint32_t w, uint32_t magic, uint32_t (&q)[4]) {
  q[0] = and_or(w << 4, 0x00F000F0u, magic);
  q[1] = and_or(w, 0x00F000F0u, magic);
  q[2] = and_or(w >> 4, 0x00F000F0u, magic);
  q[3] = and_or(w >> 8, 0x00F000F0u, magic);
}

// 8-bit word -> (c0, c2), (c1, c3) with one shift and two v_and_or_b32.
__device__ __forceinline__ void unpack_w8_ao(uint32_t w, uint32_t magic, h2 (&q)[2]) {
  q[0] = sub1024(and_or(w, 0x00FF00FFu, magic));
  q[1] = sub1024(and_or(w >> 8, 0x00FF00FFu, magic));
}

// Codes in natural k order for the MFMA B operand (the x tile is then used as
// stored, with no reordering).  A byte-select puts byte i of the word, twice,
// under the f16 exponent of 1024 (the selector's byte 5 is magic's 0x64); the
// mask keeps the low nibble in the low half (1024 + c) and the high nibble in
// the high half (1024 + 16 c); one packed f16 fma, exact, maps them to
// (c_lo, c_hi).  8-bit words: bytes 2i and 2i + 1 under the exponent, then -1024.
struct Unpack4 {
  uint32_t magic;   // kMagic
  h2 scale;         // (1, 1/16)
};
__device__ __forceinline__ u4 unpack4_natural(uint32_t w, const Unpack4& u) {
  const h2 off = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-64.0f)};
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sel = 0x05000500u | (static_cast<uint32_t>(i) << 16) | static_cast<uint32_t>(i);
    const uint32_t t = __builtin_amdgcn_perm(u.magic, w, sel) & 0x64F0640Fu;
    p[i] = as_u32(__builtin_elementwise_fma(as_h2(t), u.scale, off));
  }
  return u4{p[0], p[1], p[2], p[3]};
}
__device__ __forceinline__ u4 unpack8_natural(uint32_t w0, uint32_t w1, uint32_t magic) {
  const uint32_t sel_lo = 0x05010500u, sel_hi = 0x05030502u;
  const uint32_t p0 = __builtin_amdgcn_perm(magic, w0, sel_lo), p1 = __builtin_amdgcn_perm(magic, w0, sel_hi);
  const uint32_t p2 = __builtin_amdgcn_perm(magic, w1, sel_lo), p3 = __builtin_amdgcn_perm(magic, w1, sel_hi);
  return u4{as_u32(sub1024(p0)), as_u32(sub1024(p1)), as_u32(sub1024(p2)), as_u32(sub1024(p3))};
}

// Reorder 8 consecutive f16 activations x0..x7 (as 4 dwords (x0,x1) (x2,x3)
// (x4,x5) (x6,x7)) into the pair order of unpack_w4_off64: (x0,x4) (x1,x5) (x2,x6)
// (x3,x7).  v_perm_b32 selects bytes from two dwords.
__device__ __forceinline__ u4 perm_x_w4(u4 v) {
  u4 o;
  // __builtin_amdgcn_perm(hi, lo, sel): byte selectors 0-3 pick lo, 4-7 pick hi.
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0 from v.x lo, x4 from v.z lo)
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
  return o;
}

// Reorder two 8-bit words' activations x0..x3 | x4..x7 into (x0,x2) (x1,x3) |
// (x4,x6) (x5,x7), the pair order of unpack_w8_ao.
__device__ __forceinline__ u4 perm_x_w8(u4 v) {
  u4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x0, x2)
  o.y = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
  o.z = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x4, x6)
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x5, x7)
  return o;
}

// Sum of 8 f16 values held as 4 dwords, in f32, fixed order.
__device__ __forceinline__ float sum8_f32(u4 v) {
  const h2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  float s = __builtin_amdgcn_fdot2(as_h2(v.x), one, 0.0f, false);
  s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
  s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
  s = __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
  return s;
}

// ---------------------------------------------------------------------------
// bf16 activations.  bf16 keeps 7 mantissa bits, so the f16 tricks above change:
//  * 4-bit codes are injected under the exponent of 128 (bits 0x4300): each
//    half holds 128 + c exactly.  The offset is not subtracted per code; the
//    caller folds it into the bias term (sum x*(128 + c) = sum x*c + 128 sum x).
//    One shift per nibble position, pairs (c0, c4) (c1, c5) (c2, c6) (c3, c7)
//    as in unpack_w4_off64, so the same activation reorder (perm_x_w4) applies.
//  * 8-bit codes (up to 255, beyond what the mantissa can hold under a power
//    of two) are converted exactly: v_cvt_f32_ubyte then a packed f32 -> bf16
//    conversion, pairs in natural order (c0, c1) (c2, c3).
// ---------------------------------------------------------------------------
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
constexpr uint32_t kMagicB = 0x43004300u;

__device__ __forceinline__ b2 as_b2(uint32_t u) { return __builtin_bit_cast(b2, u); }

// 4-bit word -> (E + c0, E + c4), (E + c1, E + c5), (E + c2, E + c6),
// (E + c3, E + c7), with E the power of two whose bit pattern is `magic` in
// each half: 128 for kMagicB (bf16 pairs), 1024 for kMagic (f16 pairs).  The
// offset is left in; callers remove E * sum(x) through the group's bias.
__device__ __forceinline__ void unpack_w4_off(uint32_t w, uint32_t magic, uint32_t (&q)[4]) {
  q[0] = and_or(w, 0x000F000Fu, magic);
  q[1] = and_or(w >> 4, 0x000F000Fu, magic);
  q[2] = and_or(w >> 8, 0x000F000Fu, magic);
  q[3] = and_or(w >> 12, 0x000F000Fu, magic);
}

// ---------------------------------------------------------------------------
// int8 activations: per-row symmetric quantization, taken in f32 (each integer
// decision as the reference computation takes it): r = 127 / max|x| (0 for an
// all-zero row), code = clamp(rint(x * r), -127, 127).
// ---------------------------------------------------------------------------
// Largest |x| over 8 f16 activations (4 dwords), in f32.
__device__ __forceinline__ float absmax8_f16(u4 v) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 h = as_h2(d[i]);
    m = fmaxf(m, fmaxf(fabsf(static_cast<float>(h.x)), fabsf(static_cast<float>(h.y))));
  }
  return m;
}

// int8 code of one activation: clamp(rint(x * r), -127, 127), product and
// rounding (to nearest, ties to even) in f32.
__device__ __forceinline__ int quant_i8(float x, float r) {
  const float p = __builtin_rintf(x * r);
  return static_cast<int>(fminf(fmaxf(p, -127.0f), 127.0f));
}

__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(c) & 0xFFu) << 16) | ((static_cast<uint32_t>(d) & 0xFFu) << 24);
}

// Quantize one 16-byte chunk (8 f16 activations x0..x7) into two dwords of
// int8 codes in the byte order of the code unpack: 4-bit words split into
// even codes (x0, x2, x4, x6) and odd codes (x1, x3, x5, x7); 8-bit words hold
// four codes in natural order (x0..x3 | x4..x7).  Adds the codes to `sum`.
template <int BITS>
__device__ __forceinline__ void quant_chunk_i8(u4 v, float r, uint32_t& a, uint32_t& b, int& sum) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  int q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 h = as_h2(d[i]);
    q[2 * i] = quant_i8(static_cast<float>(h.x), r);
    q[2 * i + 1] = quant_i8(static_cast<float>(h.y), r);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += q[i];
  if constexpr (BITS == 4) {
    a = pack_i8x4(q[0], q[2], q[4], q[6]);
    b = pack_i8x4(q[1], q[3], q[5], q[7]);
  } else {
    a = pack_i8x4(q[0], q[1], q[2], q[3]);
    b = pack_i8x4(q[4], q[5], q[6], q[7]);
  }
}

// Byte i of w as an f32 integer (v_cvt_f32_ubyte<i>).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
  return static_cast<float>((w >> (8 * I)) & 0xFFu);
}

// Two f32 values -> packed bf16 pair (a low, b high), round to nearest even
// (exact for the small integers it is used on).
__device__ __forceinline__ uint32_t pack_bf16_pair(float a, float b) {
  const b2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// 8-bit word -> exact bf16 codes (c0, c1), (c2, c3).
__device__ __forceinline__ void unpack_w8_bf16(uint32_t w, uint32_t (&q)[2]) {
  q[0] = pack_bf16_pair(ubyte_f32<0>(w), ubyte_f32<1>(w));
  q[1] = pack_bf16_pair(ubyte_f32<2>(w), ubyte_f32<3>(w));
}

// 4-bit word -> exact bf16 codes in natural order (c0, c1), (c2, c3), (c4, c5), (c6, c7).
__device__ __forceinline__ u4 unpack4_bf16_natural(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  return u4{pack_bf16_pair(ubyte_f32<0>(lo), ubyte_f32<0>(hi)),
            pack_bf16_pair(ubyte_f32<1>(lo), ubyte_f32<1>(hi)),
            pack_bf16_pair(ubyte_f32<2>(lo), ubyte_f32<2>(hi)),
            pack_bf16_pair(ubyte_f32<3>(lo), ubyte_f32<3>(hi))};
}

// 8-bit words w0 (codes 0..3), w1 (codes 4..7) -> exact bf16 codes in natural order.
__device__ __forceinline__ u4 unpack8_bf16_natural(uint32_t w0, uint32_t w1) {
  uint32_t a[2], b[2];
  unpack_w8_bf16(w0, a);
  unpack_w8_bf16(w1, b);
  return u4{a[0], a[1], b[0], b[1]};
}

// Sum of 8 bf16 values held as 4 dwords, in f32, fixed order.
__device__ __forceinline__ float sum8_f32_bf16(u4 v) {
  const b2 one = as_b2(0x3F803F80u);
  float s = __builtin_amdgcn_fdot2_f32_bf16(as_b2(v.x), one, 0.0f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_b2(v.y), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_b2(v.z), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_b2(v.w), one, s, false);
  return s;
}

// Sum of 8 activations of either type (XB: bf16), in f32.
template <bool XB>
__device__ __forceinline__ float sum8_act(u4 v) {
  if constexpr (XB) {
    return sum8_f32_bf16(v);
  } else {
    return sum8_f32(v);
  }
}

// Round-to-nearest-even f32 -> f16 bits, of the f32 value itself.  The empty
// asm makes v opaque: without it the compiler folds a preceding f32 add/fma
// and this conversion into one v_fma_mixlo_f16, which rounds the exact sum
// straight to f16 -- a different (single) rounding that differs whenever the
// f32 rounding lands exactly on an f16 tie.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  asm("" : "+v"(v));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Round-to-nearest-even f32 -> bf16 bits; NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// f32 -> stored activation-type bits (XB: bf16, else f16), round to nearest even.
template <bool XB>
__device__ __forceinline__ uint16_t f32_to_act_bits(float v) {
  if constexpr (XB) {
    return f32_to_bf16_bits(v);
  } else {
    return f32_to_f16_bits(v);
  }
}

}  // namespace mxq
