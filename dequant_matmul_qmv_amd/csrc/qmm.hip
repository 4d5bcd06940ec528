// qmm: fused dequant + GEMM for prefill-sized M on gfx950 MFMA.
//
// y[m, n] = sum_g ( s[n,g] * P_g[m,n] + b[n,g] * X_g[m] ),
//   P_g[m,n] = sum_{k in g} x[m,k] * q[n,k],   X_g[m] = sum_{k in g} x[m,k]
// which is the dequant -> matmul of mlxcel #574 ("The blocker") rewritten with
// the zero-point decomposition that issue cites ("Upstream status refresh":
// a quantized matmul becomes a plain matmul plus zero-point arithmetic).
//
// Why this form: rounding each dequantized weight to f16 before an f16 MFMA
// costs ~2^-12 relative per weight, which over K = 8192 breaks the
// 2e-3 (1 + |y|) tolerance.  Codes (0..255) and x are exact in f16 and their
// products exact in f32, so P_g comes out of the MFMA with f32 accumulation
// only; the scale is applied per group in f32 on the VALU.
//
// The bias term sum_g b[n,g] X_g[m] is itself a small GEMM over the group
// index, run on the matrix cores every 16 groups as bf16 MFMAs with K = 16
// groups: X_g (f32) is split exactly into three bf16 parts (24 bits), b is
// exact in bf16 (bf16 scales) or split exactly into two bf16 parts (f16
// scales), and the products that matter at f32 precision are accumulated
// straight into the output accumulators.  That costs 3 or 5 MFMAs per 16
// groups instead of one f32 operation per output per group.
//
// Measured on this part: VALU and MFMA work of one SIMD do not overlap (their
// times add), a 32x32x16 f16 MFMA issues every 32 cycles given two independent
// accumulators, and LDS reads run at ~150 B/clk per CU.  So the kernel keeps
// VALU work per MFMA small and gives each wave a 64 x 64 sub-tile (2 x 2 MFMA
// blocks, 32 flop per LDS byte) where the tile count allows.
//
// Tiling: a workgroup of 4 waves (2 x 2) owns a BM x BN tile of y and walks K
// in stages of 64 codes.  Per stage, x[BM x 64] (reordered into the unpack's
// pair order) and the unpacked codes q[BN x 64] go to LDS (double-buffered,
// one barrier per stage) with a padded row stride (144 B, so the MFMA operand
// reads of 32 rows hit distinct banks); the per-group x sums, scales and
// biases go to LDS rings of 32 groups.  Global loads run two stages ahead in
// registers and are never conditional (rows and stages clamped), which keeps
// the compiler's load counters exact.  Tiles are assigned so that consecutive
// tiles on one XCD (dispatch is round-robin over the 8 XCDs) share a slice
// of W, for L2 reuse.
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>

#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {
constexpr int KT = 64;            // codes per stage
constexpr int LDK = KT;           // LDS row of the x / code tiles: 64 halves (128 B), 16-byte pieces XOR-swizzled
constexpr int XRING = 24;         // groups held by the x-sum ring (a bias block + lookahead)
constexpr int XGS = XRING + 4;    // x-sum ring row stride in floats (112 B)
constexpr int SRING = 32;         // groups held by the scale / bias rings (two bias blocks)
constexpr int SBS = SRING + 4;    // scale / bias ring row stride in halves (72 B: 8-byte aligned rows, distinct banks)
constexpr int BIAS_BLOCK = 16;    // groups per bias MFMA (its K)

// Position of 16-byte piece c (8 halves) within LDS row r.  Rows are 128 B,
// so without an XOR the rows an MFMA operand read touches would share banks.
// A 16-byte read is served 16 lanes (16 consecutive rows here) at a time over
// the 64 banks, i.e. 8 distinct 16-byte bank groups for the even rows and 8
// for the odd ones: XOR with (r >> 1) & 7 spreads both sets (r & 7 left rows
// r and r + 8 on the same banks; the bank-conflict counter fell by 42 %).
__device__ __forceinline__ int swz(int r, int c) { return ((c ^ ((r >> 1) & 7)) << 3); }


typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf8 as_bf8(const u4& v) { return __builtin_bit_cast(bf8, v); }
__device__ __forceinline__ h8 as_h8(const u4& v) { return __builtin_bit_cast(h8, v); }

// upper halves of two f32 bit patterns -> one packed pair of bf16 (a low, b high)
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Exact split of f32 values into bf16 parts by truncation: v = hi + mid + lo
// with each part a bf16 value (hi keeps the top 8 significant bits, the
// remainder is exact in f32, and so on).  Returned as packed bf16 fragments.
__device__ __forceinline__ void split3_bf16(const float (&v)[8], u4& hi, u4& mid, u4& lo) {
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t u = __float_as_uint(v[t]);
    h[t] = u & 0xFFFF0000u;
    const float r1 = v[t] - __uint_as_float(h[t]);
    m[t] = __float_as_uint(r1) & 0xFFFF0000u;
    l[t] = __float_as_uint(r1 - __uint_as_float(m[t]));
  }
  hi = u4{pack_hi16(h[0], h[1]), pack_hi16(h[2], h[3]), pack_hi16(h[4], h[5]), pack_hi16(h[6], h[7])};
  mid = u4{pack_hi16(m[0], m[1]), pack_hi16(m[2], m[3]), pack_hi16(m[4], m[5]), pack_hi16(m[6], m[7])};
  lo = u4{pack_hi16(l[0], l[1]), pack_hi16(l[2], l[3]), pack_hi16(l[4], l[5]), pack_hi16(l[6], l[7])};
}

// f16 bias values -> exact two-part bf16 split (an f16 has 11 significant
// bits: 8 in hi, at most 3 in lo; bf16's exponent range covers f16's).
__device__ __forceinline__ void split2_f16_to_bf16(const u4& v, u4& hi, u4& lo) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[8], l[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint16_t bits = static_cast<uint16_t>(w[t >> 1] >> (16 * (t & 1)));
    const float f = static_cast<float>(__builtin_bit_cast(_Float16, bits));
    h[t] = __float_as_uint(f) & 0xFFFF0000u;
    l[t] = __float_as_uint(f - __uint_as_float(h[t]));
  }
  hi = u4{pack_hi16(h[0], h[1]), pack_hi16(h[2], h[3]), pack_hi16(h[4], h[5]), pack_hi16(h[6], h[7])};
  lo = u4{pack_hi16(l[0], l[1]), pack_hi16(l[2], l[3]), pack_hi16(l[4], l[5]), pack_hi16(l[6], l[7])};
}

// 4-bit codes as f16 subnormals 16c * 2^-24 = c * 2^-20, in natural k order:
// exact values, and exact products with f16 activations.  The caller
// multiplies the group's f16 scale by 2^20 (exact).  The low nibbles of all
// bytes are shifted up and masked into one word, the high nibbles masked in
// place into another, and one byte select per pair places (low, high) nibble
// of byte i under zero bytes: 7 operations per word where an exponent
// injection and a packed f16 fma take 12.
// Measured on the matrix cores: products of subnormal operands keep fewer
// low-order bits in the MFMA's sum than those of normal operands with the same
// value.  With the codes at mantissa bits 0..3 one output in 30 rounded
// differently from the exponent-injected codes; at bits 4..7, as here, about
// one in 2000 (never by more than one f16 rounding step), with the error
// against an exact f64 result unchanged to four digits.  8-bit codes fill the
// low mantissa byte and keep the exact route.
__device__ __forceinline__ u4 unpack4_subn(uint32_t w) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
  // __builtin_amdgcn_perm(a, b, sel): selectors 0-3 pick bytes of b, 4-7 of a, 0x0C a zero byte
  return u4{__builtin_amdgcn_perm(hi, lo, 0x0C040C00u), __builtin_amdgcn_perm(hi, lo, 0x0C050C01u),
            __builtin_amdgcn_perm(hi, lo, 0x0C060C02u), __builtin_amdgcn_perm(hi, lo, 0x0C070C03u)};
}
}  // namespace

// Sum of v over aligned groups of 8 lanes (4 when GS == 32), in every lane of
// the group, through DPP lane swizzles (no LDS traffic).
template <int LANES>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  if constexpr (LANES == 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return v;
}

template <int BITS, int GS, int MB, int NB>
struct QmmCfg {
  static constexpr int NT = 512;                     // 8 waves: 2 pipelines x (2 x 2)
  static constexpr int PT = 256;                     // threads of one pipeline
  static constexpr int BM = 64 * MB, BN = 64 * NB;   // workgroup tile
  static constexpr int TWM = 32 * MB, TWN = 32 * NB; // wave sub-tile
  static constexpr int WPS = KT * BITS / 32;         // words per W row per stage: 8 or 16
  static constexpr int U4R = WPS / 4;                // 16-byte chunks per W row per stage: 2 or 4
  static constexpr int CODES_U4 = 128 / BITS;        // codes per 16-byte chunk: 32 or 16
  static constexpr int XCS = BM * 8;                 // x chunks (8 halves) per stage
  static constexpr int WCS = BN * U4R;               // W chunks per stage
  static constexpr int XCH = XCS / PT;               // x chunks per thread per stage
  static constexpr int WCH = (WCS + PT - 1) / PT;    // W chunks per thread per stage
  // Ring groups: the unit of the scale / bias bookkeeping.  A group of 32 or
  // 64 codes is one ring group; a group of 128 codes is split into its two
  // stages (each scaled by, and biased with, the group's scale and bias).
  static constexpr int RGC = GS < KT ? GS : KT;      // codes per ring group
  static constexpr int RPS = KT / RGC;               // ring groups per stage: 2 or 1
  static constexpr int KSPR = RGC / 16;              // MFMA k-steps per ring group
  static constexpr int NBUF = 4;                     // stage buffers: two computed, two being staged
  static constexpr int BS = BIAS_BLOCK / RPS;        // stages per bias block: 16 or 8
  static constexpr int SBL = BN / 32;                // scale / bias load steps per block (32 rows each)
  static constexpr size_t tile_bytes = static_cast<size_t>(NBUF * (BM + BN) * LDK) * 2;
  static constexpr size_t lds_bytes = tile_bytes + static_cast<size_t>(BM * XGS) * 4 +
                                      static_cast<size_t>(2 * BN * SBS) * 2;
  static_assert(XCH >= 1 && XCS % PT == 0, "x staging");
  static_assert(BS / 2 >= 4 && BS / 2 + SBL <= BS, "scale / bias load window inside the second half of a block");
  static_assert(lds_bytes <= 160 * 1024, "LDS of one CU");
  static_assert(static_cast<size_t>(4 * 64 * 16 * MB * NB) * 4 <= tile_bytes, "pipeline reduction fits");
};

// Each workgroup runs two pipelines of four waves (2 x 2, a TWM x TWN sub-tile
// each) over the same BM x BN tile; waves w and w + 4 share a SIMD.  Pipeline
// p owns the stages t with t % 2 == p: it stages them into LDS itself and
// computes them into its own accumulators, added at the end.  In each
// iteration pipeline 0 computes and then stages, pipeline 1 stages and then
// computes, so on every SIMD one wave's MFMAs run against the other wave's
// unpack / load / LDS work; one barrier per iteration.
// XB: activations (x, y, output bias) are bf16; codes are then staged as exact
// bf16 integers and contracted with bf16 MFMAs.
template <int BITS, bool SB_BF16, int GS, int MB, int NB, bool XB>
__global__ __launch_bounds__(512) void qmm_kernel(const uint16_t* __restrict__ x,
                                                  const uint32_t* __restrict__ W,
                                                  const uint16_t* __restrict__ S,
                                                  const uint16_t* __restrict__ B,
                                                  uint16_t* __restrict__ y, const uint16_t* __restrict__ ob,
                                                  float* __restrict__ part, int M, int N, int K, int tiles_m,
                                                  int tiles_n, int splits, int nks) {
  using C = QmmCfg<BITS, GS, MB, NB>;
  constexpr int BM = C::BM, BN = C::BN, TWM = C::TWM, TWN = C::TWN, PT = C::PT;
  constexpr int XCH = C::XCH, WCH = C::WCH, U4R = C::U4R, WPS = C::WPS, RPS = C::RPS;
  constexpr int XCS = C::XCS, WCS = C::WCS;
  // 4-bit codes with f16 activations and f16 scales are staged as f16
  // subnormals (a bf16 scale times 2^20 could overflow; bf16 subnormal
  // products would leave f32's normal range)
  constexpr bool SUBN = BITS == 4 && !XB && !SB_BF16;

  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* xA = reinterpret_cast<uint16_t*>(smem);              // [NBUF][BM][LDK] x, natural k order
  uint16_t* qB = xA + C::NBUF * BM * LDK;                        // [NBUF][BN][LDK] codes as exact f16
  float* xg = reinterpret_cast<float*>(smem + C::tile_bytes);    // [BM][XGS]: x sums, ring of groups
  // this pipeline's first stage buffer (stages kt with kt % 2 == pipe use kt & 3)
  uint16_t* const xAp = xA + (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 2) * BM * LDK;
  uint16_t* const qBp = qB + (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 2) * BN * LDK;
  uint16_t* sq = reinterpret_cast<uint16_t*>(xg + BM * XGS);     // [BN][SBS]: scales, ring of groups
  uint16_t* bq = sq + BN * SBS;                                  // [BN][SBS]: biases, ring of groups

  // ---- tile assignment (XCD-aware when the tile count allows it) ---------
  // A unit is (K split, tile); with splits > 1 each unit covers nks stages and
  // writes its f32 partial tile to part[split] for a fixed-order reduction.
  const int T = tiles_m * tiles_n;
  const int units = T * splits;
  int unit = blockIdx.x;
  if ((units & 7) == 0) unit = (blockIdx.x & 7) * (units >> 3) + (blockIdx.x >> 3);
  const int split = unit / T;
  const int tile = unit - split * T;
  const int tn = tile / tiles_m;
  const int tm = tile - tn * tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int t = threadIdx.x;
  const int tl = t & (PT - 1);            // thread within its pipeline
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int pipe = wave >> 2;
  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int hi = lane >> 5;               // k half of this lane in the 32x32 MFMA operands
  const int G = K / GS;
  const int kw = K * BITS / 32;
  const int kt0 = split * nks;                 // first stage of this unit
  const int nkt = min(nks, K / KT - kt0);      // stages of this unit (>= 1)
  const int GR = nkt * RPS;                    // ring groups of this unit

  Unpack4 up4;
  up4.magic = kMagic;
  up4.scale = h2{static_cast<_Float16>(1.0f), static_cast<_Float16>(0.0625f)};

  // Loads address a wave-uniform base advanced per stage plus a 32-bit lane
  // offset fixed for the kernel (the host routes shapes whose in-tile offsets
  // would not fit in 32 bits to the qmv kernel).
  const char* xbase = reinterpret_cast<const char*>(x + static_cast<size_t>(m0) * K);
  const char* wbase = reinterpret_cast<const char*>(W + static_cast<size_t>(n0) * kw);
  const char* sbase = reinterpret_cast<const char*>(S + static_cast<size_t>(n0) * G);
  const char* bbase = reinterpret_cast<const char*>(B + static_cast<size_t>(n0) * G);
  uint32_t xoff[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tl + PT * i;
    const int row = min(m0 + (c >> 3), M - 1) - m0;  // rows past M only feed output rows past M
    xoff[i] = static_cast<uint32_t>(row * K + (c & 7) * 8) * 2u;
  }
  uint32_t woff[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = min(tl + PT * i, WCS - 1);
    const int row = min(n0 + c / U4R, N - 1) - n0;
    woff[i] = static_cast<uint32_t>(row * kw + (c % U4R) * 4) * 4u;
  }
  // real group of (global) ring group rg
  auto group_of = [&](int rg) __attribute__((always_inline)) { return GS <= KT ? rg : rg >> 1; };

  // Scales and biases move in whole bias blocks (16 ring groups): a load step
  // covers 32 tile rows x 8 pairs of ring slots, so a wave reads 8 rows x 32
  // consecutive bytes where one scale per row and stage would touch 64 rows.
  // Block b + 1 is fetched during stages BS/2 .. BS/2 + SBL - 1 of block b and
  // lands in the ring slots of block b - 1, which nothing reads any more: the
  // stores of stage kt follow, across the barriers, the computes of every
  // stage up to kt - 4 (and kt - 4 >= the last stage of block b - 1).  Block 0
  // is loaded before the main loop.  Thread tl handles slot pair tl % 8 of
  // tile row 32 * step + tl / 8.
  const int sb_p = tl & 7;
  const int rg0 = kt0 * RPS;  // global ring group of this unit's first
  // 0: one 4-byte load per pair (both groups in one aligned word), 1: one
  // 2-byte load for both slots (a 128-code group's two ring groups), 2: two
  // 2-byte loads
  int sb_mode = 2;
  if constexpr (GS > KT) {
    if ((rg0 & 1) == 0) sb_mode = 1;
  } else {
    if (((G | rg0) & 1) == 0 && ((reinterpret_cast<uintptr_t>(S) | reinterpret_cast<uintptr_t>(B)) & 3) == 0)
      sb_mode = 0;
  }
  auto sbload = [&](int blk, int lrow, uint32_t& s2, uint32_t& b2) __attribute__((always_inline)) {
    const uint32_t roff = static_cast<uint32_t>(min(n0 + lrow, N - 1) - n0) * static_cast<uint32_t>(G) * 2u;
    const char* sp = sbase + roff;
    const char* bp = bbase + roff;
    const int ga = rg0 + blk * BIAS_BLOCK + 2 * sb_p;  // global ring group of the pair's first slot
    if (sb_mode == 0) {
      const size_t go = static_cast<size_t>(min(ga, G - 2)) * 2;  // G even here
      s2 = *reinterpret_cast<const uint32_t*>(sp + go);
      b2 = *reinterpret_cast<const uint32_t*>(bp + go);
    } else if (sb_mode == 1) {
      const size_t go = static_cast<size_t>(min(group_of(ga), G - 1)) * 2;
      const uint32_t sh = *reinterpret_cast<const uint16_t*>(sp + go);
      const uint32_t bh = *reinterpret_cast<const uint16_t*>(bp + go);
      s2 = sh | (sh << 16);
      b2 = bh | (bh << 16);
    } else {
      const size_t g0 = static_cast<size_t>(min(group_of(ga), G - 1)) * 2;
      const size_t g1 = static_cast<size_t>(min(group_of(ga + 1), G - 1)) * 2;
      s2 = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(sp + g0)) |
           (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(sp + g1)) << 16);
      b2 = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(bp + g0)) |
           (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(bp + g1)) << 16);
    }
  };
  auto sbstore = [&](int blk, int lrow, uint32_t s2, uint32_t b2) __attribute__((always_inline)) {
    const int slot = (blk * BIAS_BLOCK + 2 * sb_p) & (SRING - 1);
    *reinterpret_cast<uint32_t*>(&sq[lrow * SBS + slot]) = s2;
    *reinterpret_cast<uint32_t*>(&bq[lrow * SBS + slot]) = b2;
  };

  u4 xr[XCH];
  u4 wr[WCH];
  uint32_t sv, bv;
  auto gload = [&](int kt) __attribute__((always_inline)) {
    {
      // (block kb + 1 only if this unit has one)
      const int kb = kt / C::BS, st = kt - kb * C::BS - C::BS / 2;
      if (st >= 0 && st < C::SBL && (kb + 1) * C::BS < nkt) sbload(kb + 1, 32 * st + (tl >> 3), sv, bv);
    }
    kt = kt0 + min(kt, nkt - 1);  // global stage; the tail re-reads the last one, never stored where it is read
    // the stage's offsets are wave-uniform: kept in SGPRs (the empty asm stops
    // the compiler from folding them into 64-bit per-lane pointers), so each
    // load takes the SGPR-base + 32-bit lane-offset form with no VALU add
    size_t xo = static_cast<size_t>(kt) * (KT * 2), wo = static_cast<size_t>(kt) * (WPS * 4);
    asm volatile("" : "+s"(xo), "+s"(wo));
    const char* xb = xbase + xo;
    const char* wb = wbase + wo;
#pragma unroll
    for (int i = 0; i < XCH; ++i) xr[i] = *reinterpret_cast<const u4*>(xb + xoff[i]);
#pragma unroll
    for (int i = 0; i < WCH; ++i) wr[i] = *reinterpret_cast<const u4*>(wb + woff[i]);
  };

  // registers -> LDS for stage kt: x as loaded, codes unpacked to exact f16,
  // x sums per ring group, and a block load step's scales and biases.
  // Stages past the last go to a buffer and ring slots nothing reads.
  auto lstore = [&](int kt, auto par) __attribute__((always_inline)) {
    constexpr int pb = decltype(par)::value;  // stage buffer pipe + 2 pb, i.e. kt & 3
    uint16_t* xs = xAp + pb * 2 * BM * LDK;
    uint16_t* qs = qBp + pb * 2 * BN * LDK;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tl + PT * i;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u4*>(&xs[row * LDK + swz(row, ch)]) = xr[i];
      // x sums over each ring group, over the 8 (32-code groups: 4) lanes that
      // hold one row; every lane of the group writes the same value
      const float gsum = lane_group_sum<C::RGC == 32 ? 4 : 8>(sum8_act<XB>(xr[i]));
      xg[row * XGS + (kt * RPS + (RPS == 2 ? (ch >> 2) : 0)) % XRING] = gsum;
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = min(tl + PT * i, WCS - 1);  // extra threads rewrite the last chunk
      const int row = c / U4R, c0 = (c % U4R) * (C::CODES_U4 / 8);  // first 16-byte piece
      uint16_t* dst = &qs[row * LDK];
      const uint32_t wv[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
      if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<u4*>(dst + swz(row, c0 + k)) =
              XB ? unpack4_bf16_natural(wv[k]) : SUBN ? unpack4_subn(wv[k]) : unpack4_natural(wv[k], up4);
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k)
          *reinterpret_cast<u4*>(dst + swz(row, c0 + k)) =
              XB ? unpack8_bf16_natural(wv[2 * k], wv[2 * k + 1]) : unpack8_natural(wv[2 * k], wv[2 * k + 1], up4.magic);
      }
    }
    const int kb = kt / C::BS, st = kt - kb * C::BS - C::BS / 2;
    if (st >= 0 && st < C::SBL && (kb + 1) * C::BS < nkt) sbstore(kb + 1, 32 * st + (tl >> 3), sv, bv);
  };

  f16x acc[MB][NB], P[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f, P[i][j][r] = 0.0f;

  const int arow = wm * TWM + (lane & 31);  // tile row of this lane's A operand (+ i*32)
  const int bcol = wn * TWN + (lane & 31);  // tile column of this lane's B operand / output (+ j*32)

  // Bias term for ring groups [g0, g0 + ng): acc += X^T b on the matrix cores.
  auto bias_block = [&](int g0, int ng) __attribute__((always_inline)) {
    const int gb = 8 * hi;                       // this lane's first group of the block
    const int cnt = min(max(ng - gb, 0), 8);     // valid groups among this lane's 8
    const int slot = (g0 + gb) & (SRING - 1);   // 8 consecutive slots of each ring (both
    const int xslot = (g0 + gb) % XRING;        // ring sizes are multiples of 8)
    u4 bhi[NB], blo[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint2* bp = reinterpret_cast<const uint2*>(&bq[(bcol + j * 32) * SBS + slot]);  // 8-byte aligned
      const uint2 b01 = bp[0], b23 = bp[1];
      uint32_t w[4] = {b01.x, b01.y, b23.x, b23.y};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t keep = (2 * q + 1 < cnt) ? 0xFFFFFFFFu : (2 * q < cnt ? 0x0000FFFFu : 0u);
        w[q] &= keep;  // groups past the end may hold stale ring entries
      }
      const u4 v = u4{w[0], w[1], w[2], w[3]};
      if constexpr (SB_BF16) {
        bhi[j] = v;
      } else {
        split2_f16_to_bf16(v, bhi[j], blo[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float* xp = &xg[(arow + i * 32) * XGS + xslot];
      const float4 a0 = *reinterpret_cast<const float4*>(xp);
      const float4 a1 = *reinterpret_cast<const float4*>(xp + 4);
      float xv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) xv[u] = (u < cnt) ? xv[u] : 0.0f;
      u4 xh, xm, xl;
      split3_bf16(xv, xh, xm, xl);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f16x a = acc[i][j];
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(xh), as_bf8(bhi[j]), a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(xm), as_bf8(bhi[j]), a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(xl), as_bf8(bhi[j]), a, 0, 0, 0);
        if constexpr (!SB_BF16) {
          a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(xh), as_bf8(blo[j]), a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(xm), as_bf8(blo[j]), a, 0, 0, 0);
        }
        acc[i][j] = a;
      }
    }
  };

  // This pipeline's stage kt from its LDS buffer: per ring group, P from the
  // MFMAs, acc += s * P on the VALU, and the bias MFMAs when the ring group
  // closes a block of 16.
  auto compute = [&](int kt, auto par) __attribute__((always_inline)) {
    constexpr int pb = decltype(par)::value;  // stage buffer pipe + 2 pb, i.e. kt & 3
    const uint16_t* xs = xAp + pb * 2 * BM * LDK;
    const uint16_t* qs = qBp + pb * 2 * BN * LDK;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bool first = kk % C::KSPR == 0;
      u4 a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = *reinterpret_cast<const u4*>(&xs[(arow + i * 32) * LDK + swz(arow, 2 * kk + hi)]);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = *reinterpret_cast<const u4*>(&qs[(bcol + j * 32) * LDK + swz(bcol, 2 * kk + hi)]);
      const f16x zero = {};
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          P[i][j] = XB ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[i]), as_bf8(b[j]), first ? zero : P[i][j], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(a[i]), as_h8(b[j]), first ? zero : P[i][j], 0, 0, 0);
      if (kk % C::KSPR == C::KSPR - 1) {
        const int rg = kt * RPS + kk / C::KSPR;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          // widened once: the empty asm keeps the compiler from folding the f16
          // widening into each FMA (v_fma_mix_f32, VOP3P), which issues at half
          // the rate of the two-operand v_fmac_f32 used instead
          float sc = sb_to_f32<SB_BF16>(sq[(bcol + j * 32) * SBS + (rg & (SRING - 1))]);
          if constexpr (SUBN) sc *= 0x1p20f;  // P is in units of 2^-20
          asm volatile("" : "+v"(sc));
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(sc, P[i][j][r], acc[i][j][r]);
        }
        if ((rg & (BIAS_BLOCK - 1)) == BIAS_BLOCK - 1 || rg == GR - 1) {
          const int g0 = rg & ~(BIAS_BLOCK - 1);
          bias_block(g0, rg - g0 + 1);
        }
      }
    }
  };

  // ---- prologue: scales and biases of block 0; each pipeline's first stage
  // in LDS, its second in registers
#pragma unroll
  for (int i = 0; i < C::SBL / 2; ++i) {  // 64 rows per pass over both pipelines
    uint32_t s2, b2;
    sbload(0, 64 * i + (t >> 3), s2, b2);
    sbstore(0, 64 * i + (t >> 3), s2, b2);
  }
  gload(pipe);
  lstore(pipe, std::integral_constant<int, 0>{});
  gload(pipe + 2);
  __syncthreads();

  // Iteration pr: pipeline 0 computes stage 2pr, then stages 2pr + 2 and
  // prefetches 2pr + 4; pipeline 1 stages 2pr + 3 and prefetches 2pr + 5,
  // then computes 2pr + 1.  One barrier; a single loop exit keeps the
  // compiler's wait analysis exact.
  // The staging work (the longer dependent chain of the two) runs at a raised
  // wave priority, so on each SIMD it wins issue slots over the other wave's
  // scale FMAs and LDS reads while that wave's MFMAs run (measured 2-6 %).
  // Pipeline p uses stage buffers p and p + 2 in turn; the loop runs two
  // iterations per trip so that each buffer's address is a constant offset
  // from the pipeline's first (LDS immediates instead of an add per access).
  auto iteration = [&](int pr, auto par) __attribute__((always_inline)) {
    constexpr int pb = decltype(par)::value;  // pr & 1
    const int kt = 2 * pr + pipe;
    if (pipe == 1) {
      __builtin_amdgcn_s_setprio(1);
      lstore(kt + 2, std::integral_constant<int, pb ^ 1>{});
      gload(kt + 4);
      __builtin_amdgcn_s_setprio(0);
    }
    if (kt < nkt) compute(kt, par);
    if (pipe == 0) {
      __builtin_amdgcn_s_setprio(1);
      lstore(kt + 2, std::integral_constant<int, pb ^ 1>{});
      gload(kt + 4);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
  };
  const int npair = (nkt + 1) >> 1;
  int pr = 0;
  for (; pr + 1 < npair; pr += 2) {
    iteration(pr, std::integral_constant<int, 0>{});
    iteration(pr + 1, std::integral_constant<int, 1>{});
  }
  if (pr < npair) iteration(pr, std::integral_constant<int, 0>{});

  // ---- add the two pipelines' accumulators, store -------------------------
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][MB*NB*16][64], over the stage buffers
  const int q = wave & 3;
  if (pipe == 1) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((q * MB * NB + i * NB + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  }
  __syncthreads();
  if (pipe == 1) return;
  // lane holds column n, rows 8*(r/4) + 4*(lane/32) + r%4 of each 32x32 block
  float* pout = part != nullptr ? part + static_cast<size_t>(split) * M * N : nullptr;
  if (pout == nullptr && m0 + BM <= M && n0 + BN <= N && (N & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
    // Whole tile, rows of y 16-byte aligned: the wave's results go through its
    // own part of the exchange area (each value read above before it is
    // overwritten here) and leave as 16-byte row pieces, whole 64- or
    // 128-byte row segments per group of lanes.  Stored straight from the MFMA
    // layout they would be 2 bytes per lane, half a row segment per row and
    // instruction.
    constexpr int EP = TWN + 8;               // staged row stride in halves
    constexpr int LPR = TWN / 8;              // lanes per row (16-byte pieces)
    constexpr int RPI = kWave / LPR;          // rows per store instruction
    static_assert(TWM * EP * 2 <= MB * NB * 16 * 64 * 4, "staging fits in the wave's exchange area");
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((q * MB * NB + i * NB + j) * 16 + r) * 64 + lane];
    uint16_t* ep = reinterpret_cast<uint16_t*>(red + q * MB * NB * 16 * 64);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int c = j * 32 + (lane & 31);
        const float o = ob != nullptr ? sb_to_f32<XB>(ob[n0 + wn * TWN + c]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)) * EP + c] = f32_to_act_bits<XB>(acc[i][j][r] + o);
      }
    const int pc = lane % LPR, pr = lane / LPR;
    uint16_t* yt = y + static_cast<size_t>(m0 + wm * TWM) * N + n0 + wn * TWN + 8 * pc;
#pragma unroll
    for (int qq = 0; qq < TWM / RPI; ++qq) {
      const int rr = RPI * qq + pr;
      *reinterpret_cast<u4*>(yt + static_cast<size_t>(rr) * N) = *reinterpret_cast<const u4*>(&ep[rr * EP + 8 * pc]);
    }
    return;
  }
  if (m0 + BM <= M && n0 + BN <= N && N < (1 << 26)) {
    // whole tile inside y: no bounds checks; each store takes a wave-uniform
    // row base in SGPRs and the lane's fixed 32-bit offset (4*hi rows + column)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + bcol + j * 32;
        const uint32_t loff = static_cast<uint32_t>(4 * hi * N + n);  // elements; bytes below fit in 32 bits
        const float o = (ob != nullptr && pout == nullptr) ? sb_to_f32<XB>(ob[n]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[i][j][r] + red[((q * MB * NB + i * NB + j) * 16 + r) * 64 + lane] + o;
          size_t urow = static_cast<size_t>(m0 + wm * TWM + i * 32 + 8 * (r >> 2) + (r & 3)) * N;
          asm volatile("" : "+s"(urow));
          if (pout != nullptr) {
            *reinterpret_cast<float*>(reinterpret_cast<char*>(pout + urow) + loff * 4u) = v;
          } else {
            *reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(y + urow) + loff * 2u) = f32_to_act_bits<XB>(v);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + bcol + j * 32;
      const float o = (ob != nullptr && pout == nullptr) ? sb_to_f32<XB>(ob[min(n, N - 1)]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[i][j][r] + red[((q * MB * NB + i * NB + j) * 16 + r) * 64 + lane] + o;
        const int m = m0 + wm * TWM + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m < M && n < N) {
          if (pout != nullptr) {
            pout[static_cast<size_t>(m) * N + n] = v;
          } else {
            y[static_cast<size_t>(m) * N + n] = f32_to_act_bits<XB>(v);
          }
        }
      }
    }
}

// y = RNE_f16(sum over splits of part[split] (in split order) + out_bias);
// four consecutive elements per thread (the workspace is 256-byte aligned and
// MN is a multiple of 4 on this path, checked by the host).  The column of
// the first element is taken once per step (one 64-bit remainder, not four),
// and the four results leave as one 8-byte store when y allows it.
template <bool XB>
__global__ __launch_bounds__(256) void qmm_split_reduce_kernel(const float* __restrict__ part,
                                                               const uint16_t* __restrict__ ob,
                                                               uint16_t* __restrict__ y, int64_t MN, int N,
                                                               int splits) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  const bool yvec = (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < MN; i += stride) {
    float4 v = *reinterpret_cast<const float4*>(part + i);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 u = *reinterpret_cast<const float4*>(part + static_cast<size_t>(sp) * MN + i);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    float o[4] = {v.x, v.y, v.z, v.w};
    if (ob != nullptr) {
      int c = static_cast<int>(i % N);  // column of element i; the next ones wrap to column 0 past N - 1
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] += sb_to_f32<XB>(ob[c]);
        c = c + 1 == N ? 0 : c + 1;
      }
    }
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = f32_to_act_bits<XB>(o[e]);
    if (yvec) {
      *reinterpret_cast<uint2*>(y + i) = uint2{static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16),
                                               static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[i + e] = h[e];
    }
  }
}

template <int BITS, bool SB_BF16, int GS, int MB, int NB, bool XB>
static hipError_t launch_qmm_cfg(const QmmArgs& a) {
  using C = QmmCfg<BITS, GS, MB, NB>;
  const void* kern = reinterpret_cast<const void*>(&qmm_kernel<BITS, SB_BF16, GS, MB, NB, XB>);
  hipError_t e = ensure_dynamic_lds(kern, C::lds_bytes);
  if (e != hipSuccess) return e;
  const int tiles_m = static_cast<int>((a.M + C::BM - 1) / C::BM);
  const int tiles_n = static_cast<int>((a.N + C::BN - 1) / C::BN);
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int nkt = K / KT;
  int splits = a.part != nullptr ? a.splits : 1;  // the workspace holds a.splits partial tiles
  const int nks = (nkt + splits - 1) / splits;    // stages per split
  splits = (nkt + nks - 1) / nks;                 // every split non-empty, never more than a.splits
  hipLaunchKernelGGL((qmm_kernel<BITS, SB_BF16, GS, MB, NB, XB>), dim3(tiles_m * tiles_n * splits), dim3(C::NT),
                     C::lds_bytes, a.stream, a.x, a.w, a.s, a.b, a.y, a.ob, a.part, M, N, K, tiles_m, tiles_n,
                     splits, nks);
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t MN = a.M * a.N;
  int64_t blocks = (MN / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(qmm_split_reduce_kernel<XB>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, a.stream,
                     a.part, a.ob, a.y, MN, N, splits);
  return hipGetLastError();
}

template <int MB, int NB, bool XB>
static hipError_t launch_qmm_shape_x(const QmmArgs& a) {
  const int gs = a.group_size;
  if (a.bits == 4) {
    if (a.sb_bf16) {
      return gs == 32 ? launch_qmm_cfg<4, true, 32, MB, NB, XB>(a)
                      : gs == 64 ? launch_qmm_cfg<4, true, 64, MB, NB, XB>(a) : launch_qmm_cfg<4, true, 128, MB, NB, XB>(a);
    }
    return gs == 32 ? launch_qmm_cfg<4, false, 32, MB, NB, XB>(a)
                    : gs == 64 ? launch_qmm_cfg<4, false, 64, MB, NB, XB>(a) : launch_qmm_cfg<4, false, 128, MB, NB, XB>(a);
  }
  if (a.sb_bf16) {
    return gs == 32 ? launch_qmm_cfg<8, true, 32, MB, NB, XB>(a)
                    : gs == 64 ? launch_qmm_cfg<8, true, 64, MB, NB, XB>(a) : launch_qmm_cfg<8, true, 128, MB, NB, XB>(a);
  }
  return gs == 32 ? launch_qmm_cfg<8, false, 32, MB, NB, XB>(a)
                  : gs == 64 ? launch_qmm_cfg<8, false, 64, MB, NB, XB>(a) : launch_qmm_cfg<8, false, 128, MB, NB, XB>(a);
}

template <int MB, int NB>
static hipError_t launch_qmm_shape(const QmmArgs& a) {
  return a.x_bf16 ? launch_qmm_shape_x<MB, NB, true>(a) : launch_qmm_shape_x<MB, NB, false>(a);
}

// Tile policy: 128 x 128 tiles (64 x 64 per wave) when they alone give every
// CU a tile; else, for long K, the same tiles with K split so that tiles x
// splits fills the CUs (each split at least 8 stages), the partial sums going
// through a workspace and a fixed-order reduction; else 64 x 64 tiles.
QmmTile qmm_pick_tile(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
  const int64_t big = ((M + 127) / 128) * ((N + 127) / 128);
  if (big >= dev.num_cu) return QmmTile{2, 2, 1};
  const int64_t nkt = K / 64;
  int64_t splits = (dev.num_cu + big - 1) / big;
  if (splits > nkt / 8) splits = nkt / 8;
  if (splits >= 2) {
    const int64_t nks = (nkt + splits - 1) / splits;
    return QmmTile{2, 2, static_cast<int>((nkt + nks - 1) / nks)};  // no empty split
  }
  return QmmTile{1, 1, 1};
}

hipError_t launch_split_reduce_f16(const float* part, const uint16_t* ob, uint16_t* y, int64_t M, int64_t N,
                                   int splits, hipStream_t stream) {
  const int64_t MN = M * N;
  int64_t blocks = (MN / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(qmm_split_reduce_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, part,
                     ob, y, MN, static_cast<int>(N), splits);
  return hipGetLastError();
}

hipError_t launch_qmm(const QmmArgs& a0, const DeviceInfo& dev) {
  const QmmTile tl = qmm_pick_tile(a0.M, a0.N, a0.K, dev);
  QmmArgs a = a0;
  a.part = nullptr;
  a.splits = 1;
  if (tl.mb == 1) return launch_qmm_shape<1, 1>(a);
  if (tl.splits == 1) return launch_qmm_shape<2, 2>(a);
  if ((a.M * a.N) % 4 != 0) return launch_qmm_shape<1, 1>(a);  // the reduction works in fours
  // split K: an f32 workspace [splits, M, N], the stream's cached one, or
  // under graph capture one allocated and freed inside the graph
  const size_t bytes = static_cast<size_t>(tl.splits) * static_cast<size_t>(a.M) * static_cast<size_t>(a.N) * 4;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(a.stream, &cap) != hipSuccess) {
    (void)hipGetLastError();
    cap = hipStreamCaptureStatusNone;
  }
  a.splits = tl.splits;
  if (a0.fixed_ws != nullptr) {  // the caller's workspace: no allocation, capture or not
    if (bytes > a0.fixed_ws_bytes) return hipErrorInvalidValue;  // the caller checks this first
    a.part = a0.fixed_ws;
    return launch_qmm_shape<2, 2>(a);
  }
  if (cap == hipStreamCaptureStatusNone) {
    std::lock_guard<std::mutex> lk(split_workspace_mutex());
    a.part = split_workspace_locked(dev.device, a.stream, bytes);
    if (a.part == nullptr) {
      a.splits = 1;
      return launch_qmm_shape<1, 1>(a);  // no workspace: the unsplit small-tile kernel
    }
    return launch_qmm_shape<2, 2>(a);
  }
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, bytes, a.stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    a.splits = 1;
    return launch_qmm_shape<1, 1>(a);
  }
  a.part = static_cast<float*>(ws);
  e = launch_qmm_shape<2, 2>(a);
  const hipError_t ef = hipFreeAsync(ws, a.stream);
  return e != hipSuccess ? e : ef;
}

}  // namespace mxq
