// qmm_a8: fused dequant + GEMM for prefill-sized M with int8 activations, on
// the integer matrix cores (v_mfma_i32_32x32x32_i8).
//
// This is the native-int8 route of mlxcel #574 ("Next actionable step": a
// quantized dot lowered to the hardware int8 path instead of scalar widening)
// at prefill sizes.  The activations follow the per-row symmetric scheme of
// the decode and few-row kernels (every decision in f32): r = 127 / max|x|
// (0 for an all-zero row), xq = clamp(rint(x r), -127, 127), sx = max|x| / 127,
// and the path computes the dequant-matmul of x^ = sx xq:
//
//   y[m,n] = sx[m] * sum_g ( s[n,g] P_g[m,n] + b'[n,g] X_g[m] )
//   P_g = sum_{k in g} xq[m,k] q'[n,k]       exact int32 from the MFMA
//   X_g = sum_{k in g} xq[m,k]               exact integer
//
// with q' = q for 4-bit codes (0..15 fit a signed byte) and q' = q - 128 for
// 8-bit codes (one XOR per word), the offset returning through b' = b + 128 s.
//
// A small kernel quantizes each row of x once (a workgroup per row) and writes
// xq [M][K] (bytes, in the k order of the code unpack below), the x sums X
// [M][K / RGC] (f32, exact) and sx [M] to a workspace; the GEMM then stages
// plain bytes.  P_g leaves the MFMA exact, so the only rounding before the
// scale is the per-group f32 FMA acc += s * P_g (the same VALU work as the f16
// kernel's, plus one conversion).  The bias term is a small GEMM over the
// group index, run as bf16 MFMAs every 16 groups: X_g (|X_g| < 2^14, an
// integer) splits exactly into two bf16 parts, b' into one (bf16 scales,
// 4-bit), two (f16 scales, 4-bit) or three (8-bit: b + 128 s in f32) exact
// parts; every product is exact in f32 except the one dropped (the low parts
// of both, below 2^-15 of the term).
//
// Tiling: 128 x 128 tiles, a workgroup of 8 waves (2 x 4), 64 x 32 per wave (2
// x 1 blocks of 32 x 32): two waves per SIMD, so one wave's scale FMAs issue
// while the other's MFMAs or loads wait.  K in stages of 64 codes through four
// LDS buffers; global loads run four stages ahead of their LDS store in four
// register sets (x comes from other XCDs' writes and W's first reads from
// HBM: a microsecond away, several stages of compute).  The scale
// FMAs of stage t are issued after the MFMAs of stage t + 1, so they run on
// the VALU while the matrix core works on the next stage.  Long K with too few
// tiles to occupy the GPU is split, each split writing its f32 partial tile
// (already times sx) for the fixed-order split reduction.
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {
typedef int i4v __attribute__((ext_vector_type(4)));
typedef int i16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

constexpr int A8_BM = 128, A8_BN = 128, A8_NT = 512;
constexpr int A8_MB = 2, A8_NB = 1;  // 32 x 32 blocks per wave: a 2 x 4 grid of 64 x 32 wave tiles
constexpr int A8_KT = 64;            // codes per stage (one byte each in LDS)
constexpr int A8_NBUF = 4;           // LDS stage buffers
constexpr int A8_RING = 32;          // ring groups kept for scales, biases and x sums
constexpr int A8_XGS = A8_RING + 4;  // x-sum ring row stride (f32, 144 B)
constexpr int A8_SBS = A8_RING + 8;  // scale / bias ring row stride (halves, 80 B)
constexpr int A8_BB = 16;            // ring groups per bias block (the K of one bf16 MFMA)
constexpr size_t A8_TILE_BYTES = static_cast<size_t>(A8_NBUF) * (A8_BM + A8_BN) * A8_KT;
constexpr size_t A8_XG_OFF = A8_TILE_BYTES;
constexpr size_t A8_SQ_OFF = A8_XG_OFF + static_cast<size_t>(A8_BM) * A8_XGS * 4;
constexpr size_t A8_BQ_OFF = A8_SQ_OFF + static_cast<size_t>(A8_BN) * A8_SBS * 2;
constexpr size_t A8_SX_OFF = A8_BQ_OFF + static_cast<size_t>(A8_BN) * A8_SBS * 2;
constexpr size_t A8_LDS = A8_SX_OFF + A8_BM * 4;

// Byte offset of 16-byte piece c (of 4) in LDS row r of a stage tile.  A
// 16-byte operand read is served 16 lanes (16 consecutive rows) at a time;
// with 64-byte rows, rows r and r + 4 would share banks without the XOR.
__device__ __forceinline__ int pswz(int r, int c) { return (c ^ ((r >> 2) & 3)) << 4; }

// upper halves of two f32 bit patterns -> packed bf16 pair (a low, b high)
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Exact split of f32 values into NP bf16 parts by truncation (part k keeps the
// next 8 significant bits of what the previous parts left), packed for an
// MFMA operand.  NP = 3 is exact for any f32; fewer parts are exact when the
// values have at most 8 * NP significant bits.
template <int NP>
__device__ __forceinline__ void split_bf16(const float (&v)[8], u4 (&out)[NP]) {
  float rem[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) rem[t] = v[t];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      h[t] = __float_as_uint(rem[t]) & 0xFFFF0000u;
      rem[t] = rem[t] - __uint_as_float(h[t]);
    }
    out[p] = u4{hi16_pair(h[0], h[1]), hi16_pair(h[2], h[3]), hi16_pair(h[4], h[5]), hi16_pair(h[6], h[7])};
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// Row quantization: one workgroup per row of x.  xq holds each chunk of 8
// activations as two dwords in the byte order of the code unpack (4-bit:
// even then odd activations; 8-bit: natural), xs[m][j] the integer sum of the
// codes of ring group j (RGC activations), sx[m] the row scale.  Up to K = 8192
// the row stays in registers between the two passes.  (One wave per row, four
// rows per workgroup, measured slower: 4.4-5.3 against 3.8-4.1 us at K = 2048,
// 9-10 against 6 us at K = 8192, M = 512 -- a row is then a longer serial chain
// on half as many workgroups.)
// ---------------------------------------------------------------------------
// DPP move of a float (rows outside the row mask read 0, which neither a sum
// nor a maximum of non-negative values notices)
template <int CTRL, int ROWS>
__device__ __forceinline__ float a8_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

template <int BITS, int RGC>
__global__ __launch_bounds__(256) void quant_rows_i8_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ xq,
                                                            float* __restrict__ xs, float* __restrict__ sx, int K) {
  constexpr int KEEP = 4;  // passes of 256 chunks held in registers (K <= 8192: the whole row)
  const int m = blockIdx.x;
  const u4* xr = reinterpret_cast<const u4*>(x + static_cast<size_t>(m) * K);
  const int nch = K >> 3;
  float am = 0.0f;
  u4 keep[KEEP];
#pragma unroll
  for (int i = 0; i < KEEP; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;
    keep[i] = c < nch ? xr[c] : u4{0u, 0u, 0u, 0u};
    am = fmaxf(am, absmax8_f16(keep[i]));
  }
  for (int c = static_cast<int>(threadIdx.x) + 256 * KEEP; c < nch; c += 256) am = fmaxf(am, absmax8_f16(xr[c]));
  // the wave's maximum (non-negative values) folded into lane 63 by DPP moves
  // (quad swaps, half-row and row mirrors, then row_bcast:15 / :31), no LDS
  // crossbar
  am = fmaxf(am, a8_dpp<0xB1, 0xF>(am));
  am = fmaxf(am, a8_dpp<0x4E, 0xF>(am));
  am = fmaxf(am, a8_dpp<0x141, 0xF>(am));
  am = fmaxf(am, a8_dpp<0x140, 0xF>(am));
  am = fmaxf(am, a8_dpp<0x142, 0xA>(am));
  am = fmaxf(am, a8_dpp<0x143, 0xC>(am));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 63) wmax[threadIdx.x >> 6] = am;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zr = !(amax > 0.0f);
  const float r = zr ? 0.0f : 127.0f / amax;
  if (threadIdx.x == 0) sx[m] = zr ? 0.0f : amax / 127.0f;
  constexpr int L = RGC / 8;  // lanes (chunks) per ring group
  const int GR = K / RGC;
  uint32_t* qr = xq + static_cast<size_t>(m) * (K >> 2);
  // 256 chunks per pass: ring groups never straddle passes (K is a multiple of RGC)
  for (int c0 = 0; c0 < nch; c0 += 256) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    const bool live = c < nch;
    u4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < KEEP; ++i)
      if (c0 == 256 * i) v = keep[i];
    if (c0 >= 256 * KEEP && live) v = xr[c];
    uint32_t a, b;
    int sum = 0;
    quant_chunk_i8<BITS>(v, r, a, b, sum);
    if (live) {
      qr[2 * c] = a;
      qr[2 * c + 1] = b;
    }
    // the ring group's code sum over its L aligned lanes, by DPP moves (the
    // sums are integers below 2^24: exact in f32)
    float fs = static_cast<float>(sum);
    fs += a8_dpp<0xB1, 0xF>(fs);  // quad_perm 1,0,3,2
    fs += a8_dpp<0x4E, 0xF>(fs);  // quad_perm 2,3,0,1
    if constexpr (L == 8) fs += a8_dpp<0x141, 0xF>(fs);  // row_half_mirror: the other quad of the 8
    if (live && (c % L) == 0) xs[static_cast<size_t>(m) * GR + c / L] = fs;
  }
}

// ---------------------------------------------------------------------------
// The GEMM.
// ---------------------------------------------------------------------------
template <int BITS, bool SB_BF16, int GS>
__global__ __launch_bounds__(512) void qmm_a8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xsum,
                                                     const float* __restrict__ sx, const uint32_t* __restrict__ W,
                                                     const uint16_t* __restrict__ S, const uint16_t* __restrict__ B,
                                                     uint16_t* __restrict__ y, const uint16_t* __restrict__ ob,
                                                     float* __restrict__ part, int M, int N, int K, int tiles_m,
                                                     int tiles_n, int splits, int nks) {
  constexpr int BM = A8_BM, BN = A8_BN;
  constexpr int RGC = GS < 64 ? GS : 64;   // codes per ring group
  constexpr int RPS = A8_KT / RGC;         // ring groups per stage: 2 (g32) or 1
  constexpr int WB = A8_KT * BITS / 8;     // packed code bytes per W row per stage: 32 or 64
  constexpr bool DEFER = RPS == 1;         // scale FMAs of a stage issued after the next stage's MFMAs
  // bf16 parts of b': bf16 scales with 4-bit codes are exact in one, f16 in
  // two; 8-bit codes fold 128 s into b' (an f32 value): three
  constexpr int NPB = BITS == 8 ? 3 : (SB_BF16 ? 1 : 2);

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* xt = smem;                                            // [NBUF][BM][64] x codes
  unsigned char* qt = smem + A8_NBUF * BM * A8_KT;                     // [NBUF][BN][64] weight codes
  float* xg = reinterpret_cast<float*>(smem + A8_XG_OFF);              // [BM][XGS] x sums, ring
  uint16_t* sq = reinterpret_cast<uint16_t*>(smem + A8_SQ_OFF);        // [BN][SBS] scales, ring
  uint16_t* bq = reinterpret_cast<uint16_t*>(smem + A8_BQ_OFF);        // [BN][SBS] biases, ring
  float* sxs = reinterpret_cast<float*>(smem + A8_SX_OFF);             // [BM] row scales

  // ---- tile assignment: consecutive units on one XCD share a W slice ------
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
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int hi = lane >> 5;
  const int G = K / GS;
  const int GRT = K / RGC;                   // ring groups of a whole row
  const int kt0 = split * nks;
  const int nkt = min(nks, K / A8_KT - kt0);  // stages of this unit (>= 1)
  const int GR = nkt * RPS;                   // ring groups of this unit

  if (t < BM) sxs[t] = sx[min(m0 + t, M - 1)];
  // every thread stages one 16-byte piece of x and one piece (16 codes) of W
  // per stage: tile row t >> 2, piece t & 3

  // ---- per-thread load roles (rows past M or N clamped: they only feed
  // outputs that are never stored) ------------------------------------------
  const int prow = t >> 2, pc = t & 3;
  const unsigned char* xbase = xq + static_cast<size_t>(m0) * K;
  const uint32_t xoff = static_cast<uint32_t>((min(m0 + prow, M - 1) - m0) * K + pc * 16);
  const int kwb = K * BITS / 8;  // packed bytes per W row
  const unsigned char* wbase = reinterpret_cast<const unsigned char*>(W) + static_cast<size_t>(n0) * kwb;
  const uint32_t woff = static_cast<uint32_t>((min(n0 + prow, N - 1) - n0) * kwb + pc * (2 * BITS));
  // rings: the x sums, scales and biases of a whole bias block (16 ring
  // groups) are fetched at once, when the stage that opens the block is
  // loaded: entry t + 512 q (q < 4) is row (t >> 4) + 32 q, ring group t & 15
  // of the block, so a wave reads 16 consecutive groups of each of 4 rows
  // (per stage and row, one value each would touch a cache line per lane)
  const int rgi = t & (A8_BB - 1);
  const float* xsrow[4];
  const uint16_t* srow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (t >> 4) + 32 * q;
    xsrow[q] = xsum + static_cast<size_t>(min(m0 + row, M - 1)) * GRT + kt0 * RPS;
    srow[q] = S + static_cast<size_t>(min(n0 + row, N - 1)) * G;
    brow[q] = B + static_cast<size_t>(min(n0 + row, N - 1)) * G;
  }
  auto group_of = [&](int rg) __attribute__((always_inline)) { return GS <= A8_KT ? rg : rg >> 1; };
  struct RingRegs {
    float xs[4];
    uint16_t s[4], b[4];
  };
  RingRegs rr;

  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  struct Regs {
    u4 x;
    std::conditional_t<BITS == 4, u2, u4> w;  // 16 codes
  };
  Regs R[4];  // stage kt's loads live in R[kt % 4] from four stages before its LDS store
  auto gload = [&](Regs& R, int kt) __attribute__((always_inline)) {
    const int ks = kt0 + min(kt, nkt - 1);  // past the end: re-read the last stage (stored where nothing reads)
    size_t xo = static_cast<size_t>(ks) * A8_KT, wo = static_cast<size_t>(ks) * WB;
    asm volatile("" : "+s"(xo), "+s"(wo));
    const unsigned char* xb = xbase + xo;
    const unsigned char* wb = wbase + wo;
    R.x = *reinterpret_cast<const u4*>(xb + xoff);
    R.w = *reinterpret_cast<const decltype(R.w)*>(wb + woff);
    if ((kt * RPS) % A8_BB == 0) {  // this stage opens a bias block: its ring data
      const int rg = min(kt * RPS + rgi, GR - 1);  // unit-relative; past the end clamped (never read)
      const int g = group_of(kt0 * RPS + rg);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rr.xs[q] = xsrow[q][rg];
        rr.s[q] = srow[q][g];
        rr.b[q] = brow[q][g];
      }
    }
  };
  auto lstore = [&](const Regs& R, int kt) __attribute__((always_inline)) {
    unsigned char* xd = xt + (kt & (A8_NBUF - 1)) * BM * A8_KT;
    unsigned char* qd = qt + (kt & (A8_NBUF - 1)) * BN * A8_KT;
    *reinterpret_cast<u4*>(xd + prow * A8_KT + pswz(prow, pc)) = R.x;
    u4 q;
    if constexpr (BITS == 4) {
      // 8 codes per word -> even codes (c0, c2, c4, c6) then odd (c1, c3, c5,
      // c7), the order the row quantization gives the activations
      q = u4{R.w.x & 0x0F0F0F0Fu, (R.w.x >> 4) & 0x0F0F0F0Fu, R.w.y & 0x0F0F0F0Fu, (R.w.y >> 4) & 0x0F0F0F0Fu};
    } else {
      q = R.w ^ u4{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};  // signed c - 128
    }
    *reinterpret_cast<u4*>(qd + prow * A8_KT + pswz(prow, pc)) = q;
    if ((kt * RPS) % A8_BB == 0) {
      const int slot = (kt * RPS + rgi) % A8_RING;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (t >> 4) + 32 * q;
        xg[row * A8_XGS + slot] = rr.xs[q];
        sq[row * A8_SBS + slot] = rr.s[q];
        bq[row * A8_SBS + slot] = rr.b[q];
      }
    }
  };

  constexpr int MB = A8_MB, NB = A8_NB;
  f16x acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  i16v P[2][RPS][MB][NB];  // integer products of even / odd stages

  const int arow = wm * 32 * MB + (lane & 31);  // tile row of this lane's A operand (+ 32 i)
  const int bcol = wn * 32 * NB + (lane & 31);  // tile column of this lane's B operand and outputs (+ 32 j)

  // integer products of stage kt: P[e] for ring group e of the stage
  auto mma = [&](i16v (&P)[RPS][MB][NB], int kt) __attribute__((always_inline)) {
    const unsigned char* xs = xt + (kt & (A8_NBUF - 1)) * BM * A8_KT;
    const unsigned char* qs = qt + (kt & (A8_NBUF - 1)) * BN * A8_KT;
    const i16v zero = {};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i4v a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = *reinterpret_cast<const i4v*>(xs + (arow + 32 * i) * A8_KT + pswz(arow, 2 * kk + hi));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = *reinterpret_cast<const i4v*>(qs + (bcol + 32 * j) * A8_KT + pswz(bcol, 2 * kk + hi));
      const int e = RPS == 2 ? kk : 0;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          P[e][i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], (RPS == 2 || kk == 0) ? zero : P[e][i][j],
                                                             0, 0, 0);
    }
  };

  // bias term of ring groups [g0, g0 + ng) on the matrix cores
  auto bias_block = [&](int g0, int ng) __attribute__((always_inline)) {
    const int gb = 8 * hi;                    // this lane's first group of the block
    const int cnt = min(max(ng - gb, 0), 8);  // live groups among its 8
    const int slot = (g0 + gb) % A8_RING;     // 8 consecutive slots, 16-byte aligned
    u4 bp[NB][NPB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = bcol + 32 * j;
      const u4 bv = *reinterpret_cast<const u4*>(&bq[row * A8_SBS + slot]);
      u4 sv = {0u, 0u, 0u, 0u};
      if constexpr (BITS == 8) sv = *reinterpret_cast<const u4*>(&sq[row * A8_SBS + slot]);
      const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
      const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
      float f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float v = sb_to_f32<SB_BF16>(static_cast<uint16_t>(bw[u >> 1] >> (16 * (u & 1))));
        if constexpr (BITS == 8)
          v = __builtin_fmaf(128.0f, sb_to_f32<SB_BF16>(static_cast<uint16_t>(sw[u >> 1] >> (16 * (u & 1)))), v);
        f[u] = u < cnt ? v : 0.0f;  // slots past the block end hold other groups' values
      }
      split_bf16<NPB>(f, bp[j]);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float* xp = &xg[(arow + 32 * i) * A8_XGS + slot];
      const float4 a0 = *reinterpret_cast<const float4*>(xp);
      const float4 a1 = *reinterpret_cast<const float4*>(xp + 4);
      float xv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) xv[u] = u < cnt ? xv[u] : 0.0f;
      u4 xp2[2];
      split_bf16<2>(xv, xp2);  // |X| < 2^14, an integer: exact in two parts
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f16x c = acc[i][j];
#pragma unroll
        for (int p = 0; p < NPB; ++p) {
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, xp2[0]), __builtin_bit_cast(bf8v, bp[j][p]),
                                                      c, 0, 0, 0);
          if (p < 2)  // the low part of x times the low part of b' is dropped
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, xp2[1]),
                                                        __builtin_bit_cast(bf8v, bp[j][p]), c, 0, 0, 0);
        }
        acc[i][j] = c;
      }
    }
  };

  // acc += s * P per ring group of stage kt, then the bias MFMAs when a ring
  // group closes a block of 16 (or the unit)
  auto scale = [&](const i16v (&P)[RPS][MB][NB], int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < RPS; ++e) {
      const int rg = kt * RPS + e;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        // the scale widened once, out of the compiler's sight: it would otherwise fold the
        // widening into each FMA (v_fma_mix_f32, VOP3P), which issues at half the rate of the
        // two-operand v_fmac_f32 used instead
        float sc = sb_to_f32<SB_BF16>(sq[(bcol + 32 * j) * A8_SBS + rg % A8_RING]);
        asm volatile("" : "+v"(sc));
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(sc, static_cast<float>(P[e][i][j][r]), acc[i][j][r]);
      }
      if ((rg & (A8_BB - 1)) == A8_BB - 1 || rg == GR - 1) {
        const int g0 = rg & ~(A8_BB - 1);
        bias_block(g0, rg - g0 + 1);
      }
    }
  };

  // ---- prologue: stages 0 and 1 in LDS, 2 .. 5 in registers ----------------
#pragma unroll
  for (int i = 0; i < 4; ++i) gload(R[i], i);
  lstore(R[0], 0);
  lstore(R[1], 1);
  gload(R[0], 4);
  gload(R[1], 5);
  __syncthreads();
  if constexpr (DEFER) mma(P[0], 0);

  // Step kt (four per iteration, so that register sets are named statically):
  // MFMAs of stage kt + 1 and scale FMAs of stage kt (or both of stage kt
  // when not deferred), LDS store of stage kt + 2, loads of stage kt + 6, one
  // barrier.  Every wave takes part in every barrier; a stage past the end is
  // loaded and stored (clamped) but never computed.
  const int nquad = (nkt + 3) >> 2;
  for (int qd = 0; qd < nquad; ++qd) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int kt = 4 * qd + h;
      if constexpr (DEFER) {
        if (kt + 1 < nkt) mma(P[(h + 1) & 1], kt + 1);
        if (kt < nkt) scale(P[h & 1], kt);
      } else {
        if (kt < nkt) {
          mma(P[0], kt);
          scale(P[0], kt);
        }
      }
      lstore(R[(h + 2) & 3], kt + 2);
      gload(R[(h + 2) & 3], kt + 6);
      __syncthreads();
    }
  }

  // ---- store: lane holds column bcol + 32 j, rows 8 (r / 4) + 4 hi + r % 4
  // of each 32 x 32 block; y = RNE_f16(sx acc + out_bias), or the f32 partial
  // sx acc of this split
  float* pout = part != nullptr ? part + static_cast<size_t>(split) * M * N : nullptr;
  if (pout == nullptr && m0 + BM <= M && n0 + BN <= N && (N & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
    // Whole tile, rows of y 16-byte aligned: the wave's results go through its
    // own LDS area (the stage buffers are free after the loop's last barrier)
    // and leave as 16-byte row pieces, a 64-byte row segment per four lanes,
    // instead of 2-byte stores straight from the MFMA layout.
    constexpr int TWM = 32 * MB, TWN = 32 * NB;
    constexpr int EP = TWN + 8;    // staged row stride in halves (16-byte aligned rows)
    constexpr int LPR = TWN / 8;   // lanes per row
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    static_assert(static_cast<size_t>(A8_NT / 64) * TWM * EP * 2 <= A8_TILE_BYTES, "staging fits the stage buffers");
    uint16_t* ep = reinterpret_cast<uint16_t*>(smem) + wave * TWM * EP;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      float rs[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&sxs[wm * TWM + 32 * i + 8 * q + 4 * hi]);
        rs[4 * q] = v.x;
        rs[4 * q + 1] = v.y;
        rs[4 * q + 2] = v.z;
        rs[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int c = 32 * j + (lane & 31);
        const float o = ob != nullptr ? sb_to_f32<false>(ob[n0 + wn * TWN + c]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(32 * i + 8 * (r >> 2) + 4 * hi + (r & 3)) * EP + c] = f32_to_f16_bits(acc[i][j][r] * rs[r] + o);
      }
    }
    const int pc = lane % LPR, pr = lane / LPR;
    uint16_t* yt = y + static_cast<size_t>(m0 + wm * TWM) * N + n0 + wn * TWN + 8 * pc;
#pragma unroll
    for (int q = 0; q < TWM / RPI; ++q) {
      const int rr = RPI * q + pr;
      *reinterpret_cast<u4*>(yt + static_cast<size_t>(rr) * N) = *reinterpret_cast<const u4*>(&ep[rr * EP + 8 * pc]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    float rs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(&sxs[wm * 32 * MB + 32 * i + 8 * q + 4 * hi]);
      rs[4 * q] = v.x;
      rs[4 * q + 1] = v.y;
      rs[4 * q + 2] = v.z;
      rs[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + bcol + 32 * j;
      const float o = (ob != nullptr && pout == nullptr) ? sb_to_f32<false>(ob[min(n, N - 1)]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 * MB + 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float v = acc[i][j][r] * rs[r];
        if (m < M && n < N) {
          if (pout != nullptr)
            pout[static_cast<size_t>(m) * N + n] = v;
          else
            y[static_cast<size_t>(m) * N + n] = f32_to_f16_bits(v + o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

template <int BITS, bool SB_BF16, int GS>
hipError_t launch_a8_cfg(const QmmA8Launch& L, hipStream_t stream) {
  constexpr int RGC = GS < 64 ? GS : 64;
  const void* kern = reinterpret_cast<const void*>(&qmm_a8_kernel<BITS, SB_BF16, GS>);
  hipError_t e = ensure_dynamic_lds(kern, A8_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quant_rows_i8_kernel<BITS, RGC>), dim3(static_cast<unsigned>(L.M)), dim3(256), 0, stream,
                     L.x, reinterpret_cast<uint32_t*>(L.xq), L.xsum, L.sx, L.K);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((qmm_a8_kernel<BITS, SB_BF16, GS>), dim3(static_cast<unsigned>(L.tiles_m * L.tiles_n * L.splits)),
                     dim3(A8_NT), A8_LDS, stream, L.xq, L.xsum, L.sx, L.w, L.s, L.b, L.y, L.ob, L.part, L.M, L.N,
                     L.K, L.tiles_m, L.tiles_n, L.splits, L.nks);
  e = hipGetLastError();
  if (e != hipSuccess || L.splits == 1) return e;
  return launch_split_reduce_f16(L.part, L.ob, L.y, L.M, L.N, L.splits, stream);
}

hipError_t launch_a8_dispatch(const QmmA8Launch& L, int bits, int gs, bool sb_bf16, hipStream_t stream) {
  if (bits == 4) {
    if (sb_bf16)
      return gs == 32 ? launch_a8_cfg<4, true, 32>(L, stream)
                      : gs == 64 ? launch_a8_cfg<4, true, 64>(L, stream) : launch_a8_cfg<4, true, 128>(L, stream);
    return gs == 32 ? launch_a8_cfg<4, false, 32>(L, stream)
                    : gs == 64 ? launch_a8_cfg<4, false, 64>(L, stream) : launch_a8_cfg<4, false, 128>(L, stream);
  }
  if (sb_bf16)
    return gs == 32 ? launch_a8_cfg<8, true, 32>(L, stream)
                    : gs == 64 ? launch_a8_cfg<8, true, 64>(L, stream) : launch_a8_cfg<8, true, 128>(L, stream);
  return gs == 32 ? launch_a8_cfg<8, false, 32>(L, stream)
                  : gs == 64 ? launch_a8_cfg<8, false, 64>(L, stream) : launch_a8_cfg<8, false, 128>(L, stream);
}
}  // namespace

QmmA8Plan qmm_a8_plan(int64_t M, int64_t N, int64_t K, int group_size, const DeviceInfo& dev) {
  QmmA8Plan p{};
  p.tiles_m = static_cast<int>((M + A8_BM - 1) / A8_BM);
  p.tiles_n = static_cast<int>((N + A8_BN - 1) / A8_BN);
  const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n;
  const int64_t nkt = K / A8_KT;
  int64_t splits = 1;
  if (tiles < dev.num_cu && (M * N) % 4 == 0) {
    splits = (dev.num_cu + tiles - 1) / tiles;
    if (splits > nkt / 8) splits = nkt / 8;  // at least 8 stages per split
    if (splits < 1) splits = 1;
  }
  const int64_t nks = (nkt + splits - 1) / splits;
  p.nks = static_cast<int>(nks);
  p.splits = static_cast<int>((nkt + nks - 1) / nks);  // no empty split
  const int rgc = group_size < 64 ? group_size : 64;
  p.xq_bytes = round256(static_cast<size_t>(M) * static_cast<size_t>(K));
  p.xsum_bytes = round256(static_cast<size_t>(M) * static_cast<size_t>(K / rgc) * 4);
  p.sx_bytes = round256(static_cast<size_t>(M) * 4);
  p.part_bytes = p.splits > 1 ? static_cast<size_t>(p.splits) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4 : 0;
  p.workspace_bytes = p.part_bytes + p.xq_bytes + p.xsum_bytes + p.sx_bytes;
  return p;
}

size_t qmm_a8_lds_bytes() { return A8_LDS; }

hipError_t launch_qmm_a8(const QmmA8Args& a, const DeviceInfo& dev) {
  const QmmA8Plan p = qmm_a8_plan(a.M, a.N, a.K, a.group_size, dev);
  QmmA8Launch L{};
  L.x = a.x;
  L.w = a.w;
  L.s = a.s;
  L.b = a.b;
  L.y = a.y;
  L.ob = a.ob;
  L.M = static_cast<int>(a.M);
  L.N = static_cast<int>(a.N);
  L.K = static_cast<int>(a.K);
  L.tiles_m = p.tiles_m;
  L.tiles_n = p.tiles_n;
  L.splits = p.splits;
  L.nks = p.nks;
  auto carve = [&](char* base) {
    L.part = p.part_bytes ? reinterpret_cast<float*>(base) : nullptr;
    char* q = base + p.part_bytes;
    L.xq = reinterpret_cast<uint8_t*>(q);
    L.xsum = reinterpret_cast<float*>(q + p.xq_bytes);
    L.sx = reinterpret_cast<float*>(q + p.xq_bytes + p.xsum_bytes);
  };
  // the workspace: the stream's cached buffer, or under graph capture one
  // allocated and freed inside the graph; none to be had -> hipErrorOutOfMemory
  // with nothing enqueued (the caller takes another route)
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(a.stream, &cap) != hipSuccess) {
    (void)hipGetLastError();
    cap = hipStreamCaptureStatusNone;
  }
  if (cap == hipStreamCaptureStatusNone) {
    std::lock_guard<std::mutex> lk(split_workspace_mutex());
    float* ws = split_workspace_locked(dev.device, a.stream, p.workspace_bytes);
    if (ws == nullptr) return hipErrorOutOfMemory;
    carve(reinterpret_cast<char*>(ws));
    return launch_a8_dispatch(L, a.bits, a.group_size, a.sb_bf16, a.stream);
  }
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, p.workspace_bytes, a.stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hipErrorOutOfMemory;
  }
  carve(static_cast<char*>(ws));
  e = launch_a8_dispatch(L, a.bits, a.group_size, a.sb_bf16, a.stream);
  const hipError_t ef = hipFreeAsync(ws, a.stream);
  return e != hipSuccess ? e : ef;
}

}  // namespace mxq
