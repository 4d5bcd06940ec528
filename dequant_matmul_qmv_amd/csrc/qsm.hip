// qsm: fused dequant + GEMM for a few activation rows (9 <= M <= 16, batched
// decode) on the matrix cores.
//
// The decode kernel (qmv) spends two v_dot2 lanes per code pair and activation
// row, so beyond two rows it is bound by the VALU, not by HBM.  Here the codes
// go to v_mfma_f32_16x16x32_f16 as exact f16 integers against the activation
// rows padded to 16, and the per-group scale and bias are applied in f32 in the
// zero-point form of mlxcel #574 ("Upstream status refresh"):
//     y[m, n] = sum_g ( s[n,g] * P_g[m,n] + b[n,g] * X_g[m] ),
//     P_g = sum_{k in g} x[m,k] * q[n,k],   X_g = sum_{k in g} x[m,k].
// The VALU work left is the unpack and two FMAs per output per group.
//
// Measured (lm_head-sized N, K = 2048): about 55 us for 75 MB at any M up to
// 16, i.e. ~1.4 TB/s -- flat in M, so the MFMA work is not the limit but the
// W access pattern is: one load instruction reads 32 bytes from each of 16
// rows (a quarter of their 128-byte lines), and the counters show ~1.5x the
// algorithmic bytes fetched.  The decode kernel is faster up to 8 rows (one
// launch per 8 rows, 23 us at M = 3, 52 us at M = 8) and slower beyond (two
// launches: 96 us at M = 16), so this kernel takes 9..16 rows where the
// K-split kernel below (qsmk: 4- and 8-bit codes, K a multiple of 512 up to
// 4096) does not.
//
// Mapping: a workgroup of 4 waves owns 256 rows of W; a wave owns 64 of them
// as four 16-column MFMA blocks.  Lane l works on W row (l % 16) of each block
// and, as lane group g = l / 16, on codes [16g, 16g + 16) of every 64-code
// group: one 8-byte (4-bit) or 16-byte (8-bit) load per block and group, whose
// two halves are the MFMA k-steps of the group (so no MFMA mixes two groups).
// The activations, staged once per workgroup in LDS with padded rows, supply
// the matching A fragments; rows at or past M read as zero.  Groups of 128
// codes are two 64-code groups with the same scale and bias.
#include <climits>
#include <mutex>

#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {
typedef float f4 __attribute__((ext_vector_type(4)));
constexpr int kQsmWaves = 4;
constexpr int kQsmNB = 4;                                // 16-row MFMA blocks per wave
constexpr int kQsmRows = kQsmWaves * kQsmNB * 16;        // rows of W per workgroup
constexpr int kQsmPad = 8;                               // halves of padding per staged x row

}  // namespace

size_t qsm_lds_bytes(int M, int K) {
  return static_cast<size_t>(M) * (K + kQsmPad) * 2 + static_cast<size_t>(K / 64) * 16 * 4;
}

template <int BITS, bool SB_BF16>
__global__ __launch_bounds__(256) void qsm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ W,
                                                  const uint16_t* __restrict__ S, const uint16_t* __restrict__ B,
                                                  uint16_t* __restrict__ y, const uint16_t* __restrict__ ob, int M,
                                                  int N, int K, int gshift) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int XS = K + kQsmPad;                                   // staged x row stride (halves)
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);             // [M][XS]
  float* xg = reinterpret_cast<float*>(smem + static_cast<size_t>(M) * XS * 2);  // [K/64][16] group sums
  const int G64 = K / 64;
  const int G = K >> (6 + gshift);                              // real groups per row

  // ---- stage x: one (row, 64-code group) per thread and step; rows past M
  // have zero sums (their A fragments are never read from LDS)
  for (int u = threadIdx.x; u < 16 * G64; u += 256) {
    const int m = u % 16, gi = u / 16;
    float sum = 0.0f;
    if (m < M) {
      const u4* src = reinterpret_cast<const u4*>(x + static_cast<size_t>(m) * K + gi * 64);
      u4* dst = reinterpret_cast<u4*>(xs + m * XS + gi * 64);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u4 v = src[c];
        dst[c] = v;
        sum += sum8_f32(v);
      }
    }
    xg[gi * 16 + m] = sum;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // W row within a 16-row block; x row of the A operand
  const int lg = lane >> 4;    // lane group: codes [16 lg, 16 lg + 16) of each 64-code group
  const int row0 = blockIdx.x * kQsmRows + wave * kQsmNB * 16;
  Unpack4 up4;
  up4.magic = kMagic;
  up4.scale = h2{static_cast<_Float16>(1.0f), static_cast<_Float16>(0.0625f)};
  constexpr int WPG = 64 * BITS / 32;   // words per row per 64-code group: 8 or 16
  constexpr int WPL = WPG / 4;          // words per lane per group: 2 or 4
  const int kw = K * BITS / 32;

  int rows[kQsmNB];
#pragma unroll
  for (int j = 0; j < kQsmNB; ++j) rows[j] = min(row0 + 16 * j + col, N - 1);  // tail rows re-read row N-1

  f4 acc[kQsmNB];
#pragma unroll
  for (int j = 0; j < kQsmNB; ++j) acc[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // this lane's A fragments: x row `col` (rows at or past M read row M - 1
  // and are replaced by zeros, so the LDS reads are unconditional)
  const bool xrow = col < M;
  const uint16_t* xa = xs + min(col, M - 1) * XS + 16 * lg;  // + 64 gi (+ 8 for the second step)

  // Loads of QG consecutive 64-code groups into one register set (indices
  // clamped: branch-free; groups past the end re-read the last one and are
  // given scale and bias 0 below), two sets in ping-pong.  QG = 1: deeper sets
  // (2, 4) measured slower, the access pattern rather than the bytes in flight
  // being the limit.
  constexpr int QG = 1;
  struct Ld {
    uint32_t w[QG][kQsmNB][WPL];
    uint16_t s[QG][kQsmNB], b[QG][kQsmNB];
  };
  auto load = [&](Ld& d, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int gi = min(set * QG + q, G64 - 1);
      const int gr = gi >> gshift;
#pragma unroll
      for (int j = 0; j < kQsmNB; ++j) {
        const uint32_t* p = W + static_cast<size_t>(rows[j]) * kw + gi * WPG + lg * WPL;
        if constexpr (BITS == 4) {
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          const u2 v = *reinterpret_cast<const u2*>(p);
          d.w[q][j][0] = v.x;
          d.w[q][j][1] = v.y;
        } else {
          const u4 v = *reinterpret_cast<const u4*>(p);
          d.w[q][j][0] = v.x;
          d.w[q][j][1] = v.y;
          d.w[q][j][2] = v.z;
          d.w[q][j][3] = v.w;
        }
        d.s[q][j] = S[static_cast<size_t>(rows[j]) * G + gr];
        d.b[q][j] = B[static_cast<size_t>(rows[j]) * G + gr];
      }
    }
  };
  auto compute = [&](const Ld& d, int set) __attribute__((always_inline)) {
    const u4 z = {0u, 0u, 0u, 0u};
    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int graw = set * QG + q;
      const bool live = graw < G64;
      const int gi = min(graw, G64 - 1);
      const u4 r0 = *reinterpret_cast<const u4*>(xa + gi * 64);
      const u4 r1 = *reinterpret_cast<const u4*>(xa + gi * 64 + 8);
      const u4 a0 = xrow ? r0 : z, a1 = xrow ? r1 : z;
      const float4 xsum = *reinterpret_cast<const float4*>(&xg[gi * 16 + 4 * lg]);
#pragma unroll
      for (int j = 0; j < kQsmNB; ++j) {
        u4 b0, b1;
        if constexpr (BITS == 4) {
          b0 = unpack4_natural(d.w[q][j][0], up4);
          b1 = unpack4_natural(d.w[q][j][1], up4);
        } else {
          b0 = unpack8_natural(d.w[q][j][0], d.w[q][j][1], up4.magic);
          b1 = unpack8_natural(d.w[q][j][2], d.w[q][j][3], up4.magic);
        }
        f4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a0), __builtin_bit_cast(h8, b0), zero,
                                                       0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a1), __builtin_bit_cast(h8, b1), p, 0, 0, 0);
        const float sc = live ? sb_to_f32<SB_BF16>(d.s[q][j]) : 0.0f;
        const float bi = live ? sb_to_f32<SB_BF16>(d.b[q][j]) : 0.0f;
        acc[j][0] = __builtin_fmaf(bi, xsum.x, __builtin_fmaf(sc, p[0], acc[j][0]));
        acc[j][1] = __builtin_fmaf(bi, xsum.y, __builtin_fmaf(sc, p[1], acc[j][1]));
        acc[j][2] = __builtin_fmaf(bi, xsum.z, __builtin_fmaf(sc, p[2], acc[j][2]));
        acc[j][3] = __builtin_fmaf(bi, xsum.w, __builtin_fmaf(sc, p[3], acc[j][3]));
      }
    }
  };

  // two register sets in ping-pong; a single exit keeps the load counters exact
  const int nsets = (G64 + QG - 1) / QG;
  Ld cur, alt;
  load(cur, 0);
  int st = 0;
  for (; st + 1 < nsets; st += 2) {
    load(alt, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, st);
    load(cur, st + 2);  // past the end: re-reads the last group, never counted
    __builtin_amdgcn_sched_barrier(0);
    compute(alt, st + 1);
  }
  if (st < nsets) compute(cur, st);

  // ---- store: lane holds column `col` of each block, rows 4 lg .. 4 lg + 3
#pragma unroll
  for (int j = 0; j < kQsmNB; ++j) {
    const int n = row0 + 16 * j + col;
    if (n >= N) continue;
    const float o = ob != nullptr ? sb_to_f32<false>(ob[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * lg + i;
      if (m < M) y[static_cast<size_t>(m) * N + n] = f32_to_f16_bits(acc[j][i] + o);
    }
  }
}

// ---------------------------------------------------------------------------
// qsmk: the same contraction with K split over the waves of a workgroup.
//
// Wave w of a workgroup owns codes [512 w, 512 w + 512) of every row (K =
// 512 * waves, 1 to 8 waves).  Longer K runs in chunks of 512 * waves codes,
// chunk c as grid row c (codes offset by 512 * waves * c), each writing its
// f32 partial tile [c][m][n] for a fixed-order reduction kernel to add.  Its
// activation fragments for that slice
// (16 rows x 512 codes, rows at or past M zero) and their per-group sums stay
// in registers for the whole kernel.  The workgroup walks blocks of 16 W rows
// with a grid stride; for each block a wave
//  * loads its slice of the 16 rows with whole-line reads: each instruction
//    takes 4 rows, 16 lanes x 16 bytes per row (256 contiguous bytes); a
//    slice row is 256 bytes of 4-bit or 512 bytes of 8-bit codes,
//  * passes them through its own LDS region to the MFMA B layout (lane l:
//    W row l % 16, codes [16 (l / 16), +16) of each 64-code group, so the two
//    k-steps of a group never mix groups),
//  * unpacks the codes to f16 values -- 4-bit: 64 + c, exact, one shift and
//    one v_and_or_b32 per pair (the offset 64 leaves through the bias factor
//    b - 64 s), the activation fragments permuted once into the matching k
//    order; 8-bit: exact codes, a byte select under the exponent of 1024 and
//    an exact subtraction per pair, natural order --
//    runs the two v_mfma_f32_16x16x32_f16 of every group back to back and then
//    applies each group's scale and bias in f32 (s P + b X_g),
// and the waves' partial 16 x 16 tiles are added in LDS in wave order (one
// barrier per block; the buffer alternates between blocks).
namespace {
constexpr int kKsCodes = 512;                // codes per wave slice
constexpr int kKsGroups = kKsCodes / 64;     // 64-code groups per slice
constexpr int kKsMaxWaves = 8;
constexpr int kKsMaxChunks = 64;             // K up to 64 * 4096 codes
// staged row slice: 256 (4-bit) or 512 (8-bit) bytes + 16 bytes of pad
__host__ __device__ constexpr int ks_row_bytes(int bits) { return kKsCodes * bits / 8 + 16; }
constexpr int kXsRow = kKsCodes / 2 + 8;  // halves per row of the activation staging (half a slice + 16 bytes)
}  // namespace

// 4-bit word -> (64 + c0, 64 + c4), (64 + c1, 64 + c5), (64 + c2, 64 + c6),
// (64 + c3, 64 + c7) as f16 pairs: each code moved to bits 4..7 of its half,
// where under the exponent of 64 (`magic` = kMagic64) they weigh exactly 1.
// Plain code, so that the compiler emits the v_and_or_b32 itself and knows to
// insert the wait states its results need before an MFMA reads them.
__device__ __forceinline__ u4 unpack_w4_off64_mfma(uint32_t w, uint32_t magic) {
  constexpr uint32_t m = 0x00F000F0u;
  return u4{((w << 4) & m) | magic, (w & m) | magic, ((w >> 4) & m) | magic, ((w >> 8) & m) | magic};
}

size_t qsmk_lds_bytes(int waves, int bits, bool xstage) {
  const size_t blocks = static_cast<size_t>(waves) * 16 * ks_row_bytes(bits) + static_cast<size_t>(2 * waves) * 64 * 16;
  const size_t xs = xstage ? static_cast<size_t>(waves) * 16 * kXsRow * 2 : 0;  // the activations' pass, before the blocks
  return blocks > xs ? blocks : xs;
}

bool qsmk_xstage(int64_t M, bool int8_act) { return !int8_act && M >= 9; }

// XI: int8 activations -- each x row quantized in the kernel (per-row
// symmetric, f32 decisions), codes as bytes (4-bit: even then odd nibbles of
// each word; 8-bit: signed c - 128, the offset folded into the bias factor
// b + 128 s), one v_mfma_i32_16x16x64_i8 per 64-code group (exact integer dot
// products), the row scale applied at the end.
// RG ("ragged"): K a multiple of the group size but not of 512 per slice, or
// scales / biases not 16-byte aligned.  Slices may then end early or be empty:
// activation groups past K are zeros (no load), W segments past the row's end
// are loaded from the row's start instead (in bounds; their codes meet zero
// activations), and scales and biases are loaded as 2-byte values with the
// group index clamped and the values zeroed past the last group.
// XS (f16 activations, 9..16 rows): the activation slice passes through LDS in
// whole row pieces before the first block (see the prologue).
// Register budget: two waves per SIMD; three for int8 activations with 4-bit
// codes, whose variants fit it without spilling.
template <int BITS, bool SB_BF16, int GSH, int NW, bool XI, bool RG, bool XS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu((XI && BITS == 4) ? 3 : 2))) void qsmk_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ W, const uint16_t* __restrict__ S,
    const uint16_t* __restrict__ B, uint16_t* __restrict__ y, const uint16_t* __restrict__ ob, float* __restrict__ part,
    int M, int N, int K) {
  constexpr int nw = NW;
  constexpr int kKsRow = ks_row_bytes(BITS);
  constexpr int NLD = BITS;  // 16-byte loads per lane and block: 4 (4-bit) or 8 (8-bit)
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;  // A row (x row), B column (W row of the block), D column
  const int kg = lane >> 4;   // k-slot group of the operands; D rows 4 kg .. 4 kg + 3
  unsigned char* wst = smem + wave * 16 * kKsRow;                      // [16][kKsRow] this wave's codes
  float* red = reinterpret_cast<float*>(smem + nw * 16 * kKsRow);     // [2][nw][64][4] partial tiles
  // this wave's 512 codes: chunk blockIdx.y of nw slices, then slice `wave`
  const int ks0 = (static_cast<int>(blockIdx.y) * nw + wave) * kKsCodes;
  const int kw = K * BITS / 32;
  const int G = K >> (6 + GSH);
  constexpr int SBN = kKsGroups >> GSH;  // real groups per slice: 8 (g64) or 4 (g128)
  // 64-code groups of this slice inside K (ragged: fewer than 8, or none)
  const int gvalid = RG ? min(kKsGroups, (K - ks0) >> 6) : kKsGroups;

  // Loads of one block (indices clamped: branch-free; a block past the end
  // re-reads the last one and is never stored).
  struct Ld {
    u4 w[NLD];
    u4 s, b;     // SBN scales / biases of column c16 (g128: the low 8 bytes)
    uint32_t sp, bp;  // ragged: this lane's two scales / biases (groups 2 kg, 2 kg + 1 of the slice)
    uint16_t o;  // output bias of column c16 (unused without one)
  };
  const int nrb = (N + 15) >> 4;
  // this lane's 16-byte segment of the slice, per 256-byte half (8-bit slices
  // have two); ragged: a segment past the row's end reads the row's start
  const uint32_t* wlh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int wo = ks0 * BITS / 32 + 4 * c16 + 64 * h;  // words into the row
    wlh[h] = W + ((!RG || 4 * wo + 16 <= K * BITS / 8) ? wo : 0);
  }
  const int gbase = ks0 >> (6 + GSH);  // the slice's first real group
  const uint16_t* obs = ob != nullptr ? ob : S;  // without an output bias: any N readable halves
  auto load = [&](Ld& d, int rb) __attribute__((always_inline)) {
    rb = min(rb, nrb - 1);
    // instruction i: rows 4 (i % 4) + kg, the (i / 4)-th 256 bytes of the slice
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int row = min(16 * rb + 4 * (i % 4) + kg, N - 1);
      d.w[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u4*>(wlh[i / 4] + static_cast<size_t>(row) * kw));
    }
    const size_t so = static_cast<size_t>(min(16 * rb + c16, N - 1)) * G + (ks0 >> (6 + GSH));
    if constexpr (RG) {
      // 2-byte loads shared by the four lane groups: lane (c16, kg) fetches
      // the scales and biases of groups 2 kg and 2 kg + 1 of its column (index
      // clamped into the row, zero past the last group or the slice's real
      // groups); step() gathers the column's eight with shuffles (here they
      // would wait for the loads and stall the prefetch)
      const size_t sr = static_cast<size_t>(min(16 * rb + c16, N - 1)) * G;
      d.sp = 0u;
      d.bp = 0u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int u = 2 * kg + q;
        const int gi = gbase + u;
        const size_t at = sr + static_cast<size_t>(max(0, min(gi, G - 1)));
        const bool ok = u < SBN && gi < G;
        const uint32_t sv = S[at], bv = B[at];
        d.sp |= (ok ? sv : 0u) << (16 * q);
        d.bp |= (ok ? bv : 0u) << (16 * q);
      }
    } else if constexpr (GSH == 0) {
      d.s = __builtin_nontemporal_load(reinterpret_cast<const u4*>(S + so));
      d.b = __builtin_nontemporal_load(reinterpret_cast<const u4*>(B + so));
    } else {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      const u2 sv = __builtin_nontemporal_load(reinterpret_cast<const u2*>(S + so));
      const u2 bv = __builtin_nontemporal_load(reinterpret_cast<const u2*>(B + so));
      d.s = u4{sv.x, sv.y, 0u, 0u};
      d.b = u4{bv.x, bv.y, 0u, 0u};
    }
    // int8 activations: the output-bias load goes last, so that the wait for
    // a block's weights never also waits for the y store issued just before
    // the next block's loads (stores count in the same in-order counter, and
    // the compiler cannot count a store under a branch); lm_head at 3 / 8 /
    // 16 rows: 27.9 / 28.3 / 30.9 -> 26.0 / 27.8 / 29.8 us.  The f16 variants
    // ran 0.4-0.6 us slower with the same order and keep the compiler's.
    if constexpr (XI) __builtin_amdgcn_sched_barrier(0);
    d.o = obs[min(16 * rb + c16, N - 1)];  // unconditional: a load under a branch would drain the prefetch
  };

  // Workgroups walk the blocks with a grid stride.  In each round of the
  // stride, workgroup w = 32 a + 8 j + x takes block 32 a + 4 x + j: the
  // workgroups are dispatched to the 8 XCDs in turn (x = w % 8 is w's XCD),
  // so the 4 blocks that share each 128-byte line of y (64 columns) are
  // computed on one XCD at the same time, and their 32-byte pieces of the
  // line meet in that XCD's L2 before it is written back (lm_head at 8-16
  // rows about 1 us faster).  Grids that are not a multiple of 32 keep the
  // plain order.
  const int first_rb = (gridDim.x % 32 == 0) ? static_cast<int>((blockIdx.x & ~31u) | ((blockIdx.x & 7u) << 2) |
                                                                ((blockIdx.x >> 3) & 3u))
                                             : static_cast<int>(blockIdx.x);
  Ld cur, alt;
  // The first block's loads go out before the activation work below: the
  // weight stream starts while the activations are loaded and summed.  With
  // int8 activations they go out right after the activations' loads instead:
  // the wait for the activations (loads complete in order) then does not also
  // wait for the weights, and the quantization runs while they are in flight.
  if constexpr (!XI) load(cur, first_rb);

  // ---- activations of this slice, in the A layout, and the group sums of
  // the D rows this lane holds
  u4 xa[kKsGroups][2];
  float xs[kKsGroups][4];
  float sxl = 1.0f;  // row scale of x row c16 (int8 activations)
  if constexpr (XI) {
    // the row's largest |x| over all slices (a cross-wave maximum through LDS),
    // then r = 127 / max and the codes of this lane's 16 activations per group
    // in the byte order of the codes: (x0, x2, x4, x6) (x1, x3, x5, x7) ... for
    // 4-bit codes, natural for 8-bit
    const uint16_t* xp = x + static_cast<size_t>(min(c16, M - 1)) * K + ks0 + 16 * kg;
    const u4 z = {0u, 0u, 0u, 0u};
    u4 v[kKsGroups][2];
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      const bool live = c16 < M && (!RG || g < gvalid);
      v[g][0] = live ? *reinterpret_cast<const u4*>(xp + 64 * g) : z;
      v[g][1] = live ? *reinterpret_cast<const u4*>(xp + 64 * g + 8) : z;
    }
    load(cur, first_rb);
    __builtin_amdgcn_sched_barrier(0);  // the weight loads stay behind the activations' and ahead of their use
    float am = 0.0f;
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) am = fmaxf(am, fmaxf(absmax8_f16(v[g][0]), absmax8_f16(v[g][1])));
    {
      // the maximum over the row's four lane groups (lanes l, l ^ 16, l ^ 32):
      // gfx950's lane swaps, no LDS crossbar
      auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(am), __float_as_uint(am), false, false);
      am = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
      am = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    }
    float* ams = red;  // [nw][16], free until the first block
    if (kg == 0) ams[wave * 16 + c16] = am;
    __syncthreads();
    float amax = 0.0f;
    for (int w = 0; w < nw; ++w) amax = fmaxf(amax, ams[w * 16 + c16]);
    __syncthreads();
    const bool zr = !(amax > 0.0f);
    const float r = zr ? 0.0f : 127.0f / amax;
    const float sx = zr ? 0.0f : amax / 127.0f;
    typedef int v4i_ __attribute__((ext_vector_type(4)));
    const v4i_ ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const v4i_ zi = {0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      uint32_t a0, b0, a1, b1;
      int sum = 0;
      quant_chunk_i8<BITS>(v[g][0], r, a0, b0, sum);
      quant_chunk_i8<BITS>(v[g][1], r, a1, b1, sum);
      xa[g][0] = u4{a0, b0, a1, b1};
      // the group sums of the codes of the D rows this lane holds (4 kg + i),
      // straight in the D layout: the codes times a column of ones on the
      // matrix core (exact integers)
      const v4i_ d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i_, xa[g][0]), ones, zi, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[g][i] = static_cast<float>(d[i]);
    }
    sxl = sx;
  } else if constexpr (XS) {
    // XS (9..16 rows): the slice's activations (16 rows x 512, rows >= M as
    // zeros) pass through LDS in two halves of four groups: each load reads
    // two rows' whole 512-byte pieces, and the A-layout fragments are read
    // back (a row stride of kXsRow halves puts the 16 rows one read touches on
    // distinct banks).  Loaded in the A layout directly, every instruction
    // would take half of a 128-byte line from each of 16 rows.  The area is
    // this wave's share of the whole LDS, which the blocks' code staging
    // reuses after the barrier below.  (At 2..8 rows the direct loads touch
    // few distinct rows, and the pass through LDS cost more than it saved.)
    uint16_t* xst = reinterpret_cast<uint16_t*>(smem) + wave * 16 * kXsRow;
    const u4 z = {0u, 0u, 0u, 0u};
    const int lr = lane >> 5, lc = 8 * (lane & 31);  // row of the load pair, halves into the half slice
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = 2 * p + lr;
        const int col = 256 * h + lc;  // within the slice
        const bool ok = row < M && (!RG || (col >> 6) < gvalid);
        const u4 v = *reinterpret_cast<const u4*>(x + static_cast<size_t>(min(row, M - 1)) * K + (ok ? ks0 + col : 0));
        *reinterpret_cast<u4*>(xst + row * kXsRow + lc) = ok ? v : z;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = 4 * h + q;
        const uint16_t* xr = xst + c16 * kXsRow + 64 * q + 16 * kg;
        const u4 v0 = *reinterpret_cast<const u4*>(xr);
        const u4 v1 = *reinterpret_cast<const u4*>(xr + 8);
        // k slots in the order of the code unpack: 4-bit pairs (x0, x4)
        // (x1, x5) ..., 8-bit natural order
        xa[g][0] = BITS == 4 ? perm_x_w4(v0) : v0;
        xa[g][1] = BITS == 4 ? perm_x_w4(v1) : v1;
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();  // every wave's fragments read before any block's codes land in LDS
  } else {
    const uint16_t* xp = x + static_cast<size_t>(min(c16, M - 1)) * K + ks0 + 16 * kg;
    const u4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      const bool in_k = !RG || g < gvalid;
      const u4 v0 = in_k ? *reinterpret_cast<const u4*>(xp + 64 * g) : z;
      const u4 v1 = in_k ? *reinterpret_cast<const u4*>(xp + 64 * g + 8) : z;
      // k slots in the order of the code unpack: 4-bit pairs (x0, x4)
      // (x1, x5) ..., 8-bit natural order
      xa[g][0] = BITS == 4 ? perm_x_w4(c16 < M ? v0 : z) : (c16 < M ? v0 : z);
      xa[g][1] = BITS == 4 ? perm_x_w4(c16 < M ? v1 : z) : (c16 < M ? v1 : z);
    }
  }
  if constexpr (!XI) {
    // X_g of the D rows this lane holds (4 kg + i), straight in the D layout:
    // the activation fragments times a column of ones on the matrix core
    // (exact products, f32 sums)
    const u4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      const f4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
      f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][0]), __builtin_bit_cast(h8, ones), z4,
                                                    0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][1]), __builtin_bit_cast(h8, ones), d, 0, 0,
                                                 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[g][i] = d[i];
    }
  }

  uint32_t magic = BITS == 4 ? kMagic64 : kMagic;
  asm volatile("" : "+v"(magic));  // opaque to the compiler: the unpack becomes v_and_or_b32 / v_bfi_b32

  int par = 0;
  auto step = [&](const Ld& d, int rb) __attribute__((always_inline)) {
    // codes to this wave's LDS region (row 4 (i % 4) + kg, bytes 256 (i / 4) +
    // 16 c16 .. of the slice)
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      *reinterpret_cast<u4*>(wst + (4 * (i % 4) + kg) * kKsRow + 256 * (i / 4) + 16 * c16) = d.w[i];
    __builtin_amdgcn_wave_barrier();
    uint32_t sw[4] = {d.s.x, d.s.y, d.s.z, d.s.w};
    uint32_t bw[4] = {d.b.x, d.b.y, d.b.z, d.b.w};
    if constexpr (RG) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // groups 2k, 2k + 1 come from lane group k
        sw[k] = static_cast<uint32_t>(__shfl(static_cast<int>(d.sp), c16 + 16 * k));
        bw[k] = static_cast<uint32_t>(__shfl(static_cast<int>(d.bp), c16 + 16 * k));
      }
    }
    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // all groups' MFMAs first, each into its own registers, so that the
    // matrix core runs them back to back while the codes of the next group
    // are unpacked; then the scale and bias per group, in group order
    typedef int v4i __attribute__((ext_vector_type(4)));
    f4 p[kKsGroups];
    v4i pq[kKsGroups];  // int8 activations: the exact integer tiles, converted after the last MFMA
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      if constexpr (BITS == 8 && XI) {
        // codes [16 kg, 16 kg + 16) of the group as signed bytes c - 128 (one
        // XOR per word; the offset returns through the bias factor b + 128 s),
        // natural order, as the activation codes
        const u4 wv = *reinterpret_cast<const u4*>(wst + c16 * kKsRow + 64 * g + 16 * kg);
        const v4i b = {static_cast<int>(wv.x ^ 0x80808080u), static_cast<int>(wv.y ^ 0x80808080u),
                       static_cast<int>(wv.z ^ 0x80808080u), static_cast<int>(wv.w ^ 0x80808080u)};
        const v4i zi = {0, 0, 0, 0};
        pq[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xa[g][0]), b, zi, 0, 0, 0);
        continue;
      } else if constexpr (BITS == 8) {
        // codes [16 kg, 16 kg + 16) of the group: 16 bytes, natural order,
        // each byte under the f16 exponent of 1024 then 1024 subtracted (exact)
        const u4 wv = *reinterpret_cast<const u4*>(wst + c16 * kKsRow + 64 * g + 16 * kg);
        const u4 b0 = unpack8_natural(wv.x, wv.y, magic);
        const u4 b1 = unpack8_natural(wv.z, wv.w, magic);
        p[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][0]), __builtin_bit_cast(h8, b0),
                                                      zero, 0, 0, 0);
        p[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][1]), __builtin_bit_cast(h8, b1),
                                                      p[g], 0, 0, 0);
        continue;
      }
      const u2 wv = *reinterpret_cast<const u2*>(wst + c16 * kKsRow + 32 * g + 8 * kg);
      if constexpr (XI) {
        // codes as bytes, even then odd nibbles of each word (the order of
        // the activation codes); exact int32 dot products, at most 64 * 127 *
        // 15 in magnitude, so exact in f32 as well
        const v4i b = {static_cast<int>(wv.x & 0x0F0F0F0Fu), static_cast<int>((wv.x >> 4) & 0x0F0F0F0Fu),
                       static_cast<int>(wv.y & 0x0F0F0F0Fu), static_cast<int>((wv.y >> 4) & 0x0F0F0F0Fu)};
        const v4i zi = {0, 0, 0, 0};
        pq[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xa[g][0]), b, zi, 0, 0, 0);
      } else {
        const u4 b0 = unpack_w4_off64_mfma(wv.x, magic);  // 64 + c, exact
        const u4 b1 = unpack_w4_off64_mfma(wv.y, magic);
        p[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][0]), __builtin_bit_cast(h8, b0),
                                                      zero, 0, 0, 0);
        p[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[g][1]), __builtin_bit_cast(h8, b1),
                                                      p[g], 0, 0, 0);
      }
    }
    f4 acc = zero;
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
      const int r = g >> GSH;
      // scale and bias widened once: the empty asm keeps the compiler from
      // folding the f16 widening into each of the FMAs below (v_fma_mix_f32,
      // VOP3P, issued at half the rate of the two-operand v_fmac_f32)
      float sc = sb_to_f32<SB_BF16>(static_cast<uint16_t>(sw[r >> 1] >> (16 * (r & 1))));
      asm volatile("" : "+v"(sc));
      float bi = sb_to_f32<SB_BF16>(static_cast<uint16_t>(bw[r >> 1] >> (16 * (r & 1))));
      if constexpr (XI && BITS == 8) bi = __builtin_fmaf(128.0f, sc, bi);  // signed codes c - 128
      if constexpr (!XI && BITS == 4) bi = __builtin_fmaf(-64.0f, sc, bi);  // codes 64 + c
      asm volatile("" : "+v"(bi));
      if constexpr (XI)
        p[g] = f4{static_cast<float>(pq[g][0]), static_cast<float>(pq[g][1]), static_cast<float>(pq[g][2]),
                  static_cast<float>(pq[g][3])};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(bi, xs[g][i], __builtin_fmaf(sc, p[g][i], acc[i]));
    }
    // add the waves' tiles: wave w finishes D rows 4 kg + i for i = w, w + nw, ...
    *reinterpret_cast<f4*>(red + ((par * nw + wave) * 64 + lane) * 4) = acc;
    __syncthreads();
    const int n = 16 * rb + c16;
    const float o = ob != nullptr ? sb_to_f32<false>(d.o) : 0.0f;
    for (int i = wave; i < 4; i += nw) {
      float v = red[((par * nw) * 64 + lane) * 4 + i];
#pragma unroll
      for (int w = 1; w < nw; ++w) v += red[((par * nw + w) * 64 + lane) * 4 + i];
      const int m = 4 * kg + i;
      // the row scale of D row m from lane m (i is wave-uniform but not a
      // constant: an array indexed by it would live in scratch memory)
      const float sxi = XI ? __shfl(sxl, m) : 1.0f;
      if (m < M && n < N) {
        if (part != nullptr)  // one K chunk's f32 partial, [chunk][m][n]
          part[(static_cast<size_t>(blockIdx.y) * M + m) * N + n] = v;
        else
          y[static_cast<size_t>(m) * N + n] = f32_to_f16_bits((XI ? v * sxi : v) + o);
      }
    }
    par ^= 1;
  };

  // Two register sets in ping-pong over this workgroup's blocks (the first
  // block is in cur); a single loop exit keeps the load counters exact.
  const int stride = gridDim.x;
  int rb = first_rb;
  for (; rb + stride < nrb; rb += 2 * stride) {
    load(alt, rb + stride);
    __builtin_amdgcn_sched_barrier(0);
    step(cur, rb);
    load(cur, rb + 2 * stride);
    __builtin_amdgcn_sched_barrier(0);
    step(alt, rb + stride);
  }
  if (rb < nrb) step(cur, rb);
}

bool qsmk_ragged(int64_t K, const void* s, const void* b) {
  return K % kKsCodes != 0 || (reinterpret_cast<uintptr_t>(s) & 15) != 0 || (reinterpret_cast<uintptr_t>(b) & 15) != 0;
}

bool qsmk_split(int64_t K, int* waves, int* chunks) {
  if (K < 64 || K % 64 != 0) return false;
  if (K % kKsCodes != 0) {
    if (K < kKsCodes) return false;  // a single partial slice: the other kernels
    // ragged: ceil(K / 512) slices over the fewest chunks of at most
    // kKsMaxWaves waves (the last slices may end early or be empty)
    const int64_t S = (K + kKsCodes - 1) / kKsCodes;
    const int64_t c = (S + kKsMaxWaves - 1) / kKsMaxWaves;
    if (c > kKsMaxChunks) return false;
    *chunks = static_cast<int>(c);
    *waves = static_cast<int>((S + c - 1) / c);
    return true;
  }
  const int64_t S = K / kKsCodes;  // 512-code slices
  // the fewest chunks of at most kKsMaxWaves slices each that divide S
  for (int64_t c = (S + kKsMaxWaves - 1) / kKsMaxWaves; c <= S && c <= kKsMaxChunks; ++c) {
    if (S % c == 0) {
      *waves = static_cast<int>(S / c);
      *chunks = static_cast<int>(c);
      return true;
    }
  }
  return false;
}

bool qsmk_shape(int64_t M, int64_t N, int64_t K, int bits, int group_size, bool chunks_ok, const DeviceInfo& dev) {
  if ((bits != 4 && bits != 8) || M < 2 || M > 16 || (group_size != 64 && group_size != 128) || K % group_size != 0)
    return false;
  int nw = 0, chunks = 0;
  if (!qsmk_split(K, &nw, &chunks)) return false;
  if (chunks > 1 && (!chunks_ok || (M * N) % 4 != 0 || N > INT_MAX / 16)) return false;
  // at least one block of 16 rows per compute unit, counting every chunk
  // (smaller N stays on qmv)
  return (N + 15) / 16 * chunks >= static_cast<int64_t>(dev.num_cu);
}

namespace {
template <int BITS, bool SB_BF16, int GSH, bool XI, bool RG, bool XS>
const void* qsmk_ptr_x(int nw) {
  switch (nw) {
    case 1: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 1, XI, RG, XS>);
    case 2: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 2, XI, RG, XS>);
    case 3: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 3, XI, RG, XS>);
    case 4: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 4, XI, RG, XS>);
    case 5: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 5, XI, RG, XS>);
    case 6: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 6, XI, RG, XS>);
    case 7: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 7, XI, RG, XS>);
    default: return reinterpret_cast<const void*>(&qsmk_kernel<BITS, SB_BF16, GSH, 8, XI, RG, XS>);
  }
}
// activations: 0 f16 loaded in the A layout, 1 int8 (quantized in the
// kernel), 2 f16 staged through LDS
template <int BITS, bool SB_BF16, int GSH, bool RG>
const void* qsmk_ptr_a(int nw, int act) {
  return act == 1   ? qsmk_ptr_x<BITS, SB_BF16, GSH, true, RG, false>(nw)
         : act == 2 ? qsmk_ptr_x<BITS, SB_BF16, GSH, false, RG, true>(nw)
                    : qsmk_ptr_x<BITS, SB_BF16, GSH, false, RG, false>(nw);
}
template <bool SB_BF16, int GSH, bool RG>
const void* qsmk_ptr_r(int nw, int bits, int act) {
  return bits == 8 ? qsmk_ptr_a<8, SB_BF16, GSH, RG>(nw, act) : qsmk_ptr_a<4, SB_BF16, GSH, RG>(nw, act);
}
template <bool SB_BF16, int GSH>
const void* qsmk_ptr(int nw, int bits, int act, bool rg) {
  return rg ? qsmk_ptr_r<SB_BF16, GSH, true>(nw, bits, act) : qsmk_ptr_r<SB_BF16, GSH, false>(nw, bits, act);
}
}  // namespace

hipError_t launch_qsmk(const QmvArgs& a, int M, const DeviceInfo& dev) {
  int nw = 0, chunks = 0;
  if (!qsmk_split(a.K, &nw, &chunks)) return hipErrorInvalidValue;  // the caller checked qsmk_shape
  const bool g128 = a.glog2 == 7;
  const bool xi = a.act == 2;  // int8 activations (quantized in the kernel)
  if (chunks > 1 && xi) return hipErrorInvalidValue;
  const bool xstage = qsmk_xstage(M, xi);
  const size_t lds = qsmk_lds_bytes(nw, a.bits, xstage);
  const bool rg = qsmk_ragged(a.K, a.s, a.b);
  const int act = xi ? 1 : xstage ? 2 : 0;
  const void* kern = a.sb_bf16 ? (g128 ? qsmk_ptr<true, 1>(nw, a.bits, act, rg) : qsmk_ptr<true, 0>(nw, a.bits, act, rg))
                               : (g128 ? qsmk_ptr<false, 1>(nw, a.bits, act, rg) : qsmk_ptr<false, 0>(nw, a.bits, act, rg));
  if (lds > 65536) {  // 8 waves of 8-bit slices
    const hipError_t e = ensure_dynamic_lds(kern, lds);
    if (e != hipSuccess) return e;
  }
  // two workgroups per CU; three with int8 activations and 4-bit codes, whose
  // variants fit three waves per SIMD without spilling (lm_head, 4-8 rows: 1 us
  // faster; the f16 and 8-bit variants would spill at that register budget)
  const int occ = occupancy_blocks(kern, 64 * nw, lds);
  const int want = (xi && a.bits == 4) ? 3 : 2;
  const int per_cu = occ < want ? occ : want;
  const int64_t nrb = (a.N + 15) / 16;
  const int64_t cap = (static_cast<int64_t>(dev.num_cu) * per_cu + chunks - 1) / chunks;  // workgroups per chunk
  const unsigned gx = static_cast<unsigned>(nrb < cap ? nrb : cap);
  const uint16_t* xp = a.x;
  const uint32_t* wp = a.w;
  const uint16_t* sp = a.s;
  const uint16_t* bp = a.b;
  uint16_t* yp = a.y;
  const uint16_t* obp = a.ob;
  int Mi = M, Ni = static_cast<int>(a.N), Ki = static_cast<int>(a.K);
  if (chunks == 1) {
    float* partp = nullptr;
    void* args[] = {&xp, &wp, &sp, &bp, &yp, &obp, &partp, &Mi, &Ni, &Ki};
    return hipLaunchKernel(kern, dim3(gx), dim3(64 * nw), args, lds, a.stream);
  }
  // K in chunks: f32 partial tiles [chunks, M, N] in the stream's split
  // workspace, then the fixed-order sum, the output bias and the f16 rounding
  const size_t bytes = static_cast<size_t>(chunks) * static_cast<size_t>(M) * static_cast<size_t>(a.N) * 4;
  const uint16_t* no_ob = nullptr;  // the output bias is added once, by the reduction
  if (a.fixed_ws != nullptr) {  // the caller's workspace: no allocation
    if (bytes > a.fixed_ws_bytes) return hipErrorInvalidValue;  // the caller checks this first
    float* partp = a.fixed_ws;
    void* args[] = {&xp, &wp, &sp, &bp, &yp, &no_ob, &partp, &Mi, &Ni, &Ki};
    hipError_t e = hipLaunchKernel(kern, dim3(gx, static_cast<unsigned>(chunks)), dim3(64 * nw), args, lds, a.stream);
    if (e != hipSuccess) return e;
    return launch_split_reduce_f16(partp, obp, yp, M, a.N, chunks, a.stream);
  }
  std::lock_guard<std::mutex> lk(split_workspace_mutex());
  float* partp = split_workspace_locked(dev.device, a.stream, bytes);
  if (partp == nullptr) return hipErrorOutOfMemory;
  void* args[] = {&xp, &wp, &sp, &bp, &yp, &no_ob, &partp, &Mi, &Ni, &Ki};
  hipError_t e = hipLaunchKernel(kern, dim3(gx, static_cast<unsigned>(chunks)), dim3(64 * nw), args, lds, a.stream);
  if (e != hipSuccess) return e;
  return launch_split_reduce_f16(partp, obp, yp, M, a.N, chunks, a.stream);
}

bool qsm_shape(int64_t M, int64_t N, int64_t K, int bits, int group_size, const DeviceInfo& dev) {
  (void)bits;
  if (M < 9 || M > 16 || K % 64 != 0 || K < 64 || (group_size != 64 && group_size != 128)) return false;
  if (qsm_lds_bytes(static_cast<int>(M), static_cast<int>(K)) > dev.lds_per_block) return false;
  // enough workgroups to give every compute unit one (smaller N stays on qmv)
  return (N + kQsmRows - 1) / kQsmRows >= static_cast<int64_t>(dev.num_cu);
}

hipError_t launch_qsm(const QmvArgs& a, int M, const DeviceInfo& dev) {
  (void)dev;
  const size_t lds = qsm_lds_bytes(M, static_cast<int>(a.K));
  const void* kern = a.bits == 4 ? (a.sb_bf16 ? reinterpret_cast<const void*>(&qsm_kernel<4, true>)
                                              : reinterpret_cast<const void*>(&qsm_kernel<4, false>))
                                 : (a.sb_bf16 ? reinterpret_cast<const void*>(&qsm_kernel<8, true>)
                                              : reinterpret_cast<const void*>(&qsm_kernel<8, false>));
  if (lds > 65536) {
    hipError_t e = ensure_dynamic_lds(kern, lds);
    if (e != hipSuccess) return e;
  }
  const uint16_t* xp = a.x;
  const uint32_t* wp = a.w;
  const uint16_t* sp = a.s;
  const uint16_t* bp = a.b;
  uint16_t* yp = a.y;
  const uint16_t* obp = a.ob;
  int Mi = M, Ni = static_cast<int>(a.N), Ki = static_cast<int>(a.K), gshift = a.glog2 - 6;
  void* args[] = {&xp, &wp, &sp, &bp, &yp, &obp, &Mi, &Ni, &Ki, &gshift};
  const unsigned grid = static_cast<unsigned>((a.N + kQsmRows - 1) / kQsmRows);
  return hipLaunchKernel(kern, dim3(grid), dim3(256), args, lds, a.stream);
}

}  // namespace mxq
