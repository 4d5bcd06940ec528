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
// launches: 96 us at M = 16), so this kernel takes 9..16 rows.
//
// Mapping: a workgroup of 4 waves owns 256 rows of W; a wave owns 64 of them
// as four 16-column MFMA blocks.  Lane l works on W row (l % 16) of each block
// and, as lane group g = l / 16, on codes [16g, 16g + 16) of every 64-code
// group: one 8-byte (4-bit) or 16-byte (8-bit) load per block and group, whose
// two halves are the MFMA k-steps of the group (so no MFMA mixes two groups).
// The activations, staged once per workgroup in LDS with padded rows, supply
// the matching A fragments; rows at or past M read as zero.  Groups of 128
// codes are two 64-code groups with the same scale and bias.
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
