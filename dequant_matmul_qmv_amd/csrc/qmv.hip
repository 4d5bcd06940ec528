// qmv: fused unpack + dequant + GEMV for decode-sized M (1..8) on gfx950.
//
// y[m, n] = sum_k x[m, k] * (q[n, k] * s[n, g(k)] + b[n, g(k)])
// (mlxcel #574 "What is already in-tree": q*scale + bias; "The blocker": the
// fused kernel must not materialise the weight).  At M <= 8 every weight byte
// is used M times at most, so the kernel is bound by HBM bandwidth, and the
// whole design is about streaming W once with full-width loads while keeping
// the per-weight ALU cost low:
//
//  * A "segment" is 16 bytes of one row of W (4 words: 32 4-bit or 16 8-bit
//    codes).  All 64 lanes of a wave work on the same R rows; lane l takes
//    segments l, l+64, ... of each row, so one global_load_dwordx4 per row
//    moves 1 KiB of contiguous codes per wave.
//  * Codes become exact f16 integers (exponent injection, two per v_and_or_b32)
//    and meet the activations in v_dot2_f32_f16 with f32 accumulation.  A
//    segment never straddles a group (group_size >= 32 codes), so its scale and
//    bias are applied once per segment in f32:
//        acc += s * sum(x*q) + b * sum(x)     (zero-point form, mlxcel #574
//                                              "Upstream status refresh")
//    where sum(x) over the segment is precomputed.
//  * x is staged once per workgroup in LDS, already reordered into the pair
//    order of the unpack, laid out [m][chunk][segment] so that the 64 lanes'
//    16-byte reads hit consecutive addresses (no bank conflicts), together
//    with the per-segment sums of x.
//  * Partial sums of the R*M outputs are reduced across the wave with a
//    "transpose" butterfly: each stage halves the number of live values per
//    lane, so R*M values need (R*M - 1) + (6 - log2(R*M)) exchanges instead of
//    6*R*M.  Everything is in a fixed order: results are deterministic.
//  * Workgroups are persistent (grid-stride over row blocks) so the x staging
//    is paid once per workgroup, not once per row block.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

template <int BITS>
struct SegTraits {
  static constexpr int kCodesPerSeg = 128 / BITS;          // 32 or 16
  static constexpr int kChunksPerSeg = kCodesPerSeg * 2 / 16;  // x bytes / 16: 4 or 2
};

// LDS bytes for MT activation rows of length K.
template <int BITS>
__host__ __device__ constexpr size_t qmv_lds_bytes(int MT, int K) {
  return static_cast<size_t>(MT) * (K * BITS / 128) *
         (SegTraits<BITS>::kChunksPerSeg * 16 + 4);
}

template <int BITS, bool SB_BF16, int MT, int R>
__global__ __launch_bounds__(256) void qmv_kernel(const uint16_t* __restrict__ x,
                                                  const uint32_t* __restrict__ W,
                                                  const uint16_t* __restrict__ S,
                                                  const uint16_t* __restrict__ B,
                                                  uint16_t* __restrict__ y, int N, int K,
                                                  int glog2, int x_vec) {
  constexpr int CPS = SegTraits<BITS>::kChunksPerSeg;
  constexpr int CODES = SegTraits<BITS>::kCodesPerSeg;
  constexpr int V = R * MT;
  constexpr int VP = V <= 1 ? 1 : V <= 2 ? 2 : V <= 4 ? 4 : V <= 8 ? 8 : V <= 16 ? 16 : 32;
  static_assert(V <= 32, "too many live outputs per lane");

  extern __shared__ __align__(16) unsigned char smem[];
  const int nseg = K * BITS / 128;   // segments per row
  const int kw = K * BITS / 32;      // words per row
  const int G = K >> glog2;          // groups per row
  u4* xs = reinterpret_cast<u4*>(smem);                                     // [MT][CPS][nseg]
  float* xsum = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * CPS * nseg * 16);  // [MT][nseg]

  // ---- stage x (reordered) and its per-segment sums into LDS -------------
  for (int u = threadIdx.x; u < MT * nseg; u += blockDim.x) {
    const int m = u / nseg;
    const int seg = u - m * nseg;
    const uint16_t* xp = x + static_cast<size_t>(m) * K + seg * CODES;
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      u4 v;
      if (x_vec) {
        v = *reinterpret_cast<const u4*>(xp + 8 * c);
      } else {
        uint32_t t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          t[i] = static_cast<uint32_t>(xp[8 * c + 2 * i]) |
                 (static_cast<uint32_t>(xp[8 * c + 2 * i + 1]) << 16);
        v = u4{t[0], t[1], t[2], t[3]};
      }
      sum += sum8_f32(v);
      xs[(m * CPS + c) * nseg + seg] = (BITS == 4) ? perm_x_w4(v) : perm_x_w8(v);
    }
    xsum[m * nseg + seg] = sum;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int waves_per_block = blockDim.x >> 6;
  const int nrb = (N + R - 1) / R;
  const int jn = (nseg + kWave - 1) / kWave;

  for (int rb = blockIdx.x * waves_per_block + wave; rb < nrb; rb += gridDim.x * waves_per_block) {
    const int row0 = rb * R;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    for (int j = 0; j < jn; ++j) {
      const int seg = lane + j * kWave;
      if (seg < nseg) {
        const int grp = (seg * CODES) >> glog2;
        u4 wv[R];
        float sc[R], bi[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = min(row0 + r, N - 1);  // tail rows re-read the last row; never stored
          wv[r] = *reinterpret_cast<const u4*>(W + static_cast<size_t>(row) * kw + seg * 4);
          sc[r] = sb_to_f32<SB_BF16>(S[static_cast<size_t>(row) * G + grp]);
          bi[r] = sb_to_f32<SB_BF16>(B[static_cast<size_t>(row) * G + grp]);
        }
        // codes of the R rows, unpacked once: 16 (4-bit) or 8 (8-bit) pairs per row
        constexpr int NP = (BITS == 4) ? 16 : 8;
        h2 q[R][NP];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t wr[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (BITS == 4) {
              h2 t[4];
              unpack_w4(wr[i], t);
#pragma unroll
              for (int p = 0; p < 4; ++p) q[r][4 * i + p] = t[p];
            } else {
              h2 t[2];
              unpack_w8(wr[i], t);
              q[r][2 * i] = t[0];
              q[r][2 * i + 1] = t[1];
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          // x pairs in the same order as q: chunk c holds pairs 4c..4c+3
          uint32_t xp[NP];
#pragma unroll
          for (int c = 0; c < CPS; ++c) {
            const u4 xv = xs[(m * CPS + c) * nseg + seg];
            xp[4 * c] = xv.x;
            xp[4 * c + 1] = xv.y;
            xp[4 * c + 2] = xv.z;
            xp[4 * c + 3] = xv.w;
          }
          const float xsm = xsum[m * nseg + seg];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float d = 0.0f;
#pragma unroll
            for (int p = 0; p < NP; ++p) d = __builtin_amdgcn_fdot2(q[r][p], as_h2(xp[p]), d, false);
            acc[r][m] = __builtin_fmaf(sc[r], d, acc[r][m]);
            acc[r][m] = __builtin_fmaf(bi[r], xsm, acc[r][m]);
          }
        }
      }
    }

    // ---- transpose butterfly over the 64 lanes -------------------------
    float v[VP];
#pragma unroll
    for (int i = 0; i < VP; ++i) v[i] = (i < V) ? acc[i / MT][i % MT] : 0.0f;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      const int off = 32 >> s;
      const int live = VP >> s;  // values still live per lane before this stage
      if (live >= 2) {
        const int h = live / 2;
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
          const float send = upper ? v[i] : v[i + h];
          const float keep = upper ? v[i + h] : v[i];
          v[i] = keep + __shfl_xor(send, off, kWave);
        }
      } else {
        v[0] += __shfl_xor(v[0], off, kWave);
      }
    }
    // lane holds value index idx = sum over halving stages of bit(lane, off) * h
    constexpr int kLow = kWave / VP;  // lanes sharing one value index
    if ((lane & (kLow - 1)) == 0) {
      int idx = 0;
#pragma unroll
      for (int s = 0; s < 6; ++s) {
        const int off = 32 >> s;
        const int live = VP >> s;
        if (live >= 2 && (lane & off)) idx += live / 2;
      }
      if (idx < V) {
        const int r = idx / MT;
        const int m = idx - r * MT;
        const int row = row0 + r;
        if (row < N) y[static_cast<size_t>(m) * N + row] = f32_to_f16_bits(v[0]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launcher: picks MT/R instantiation; validation happens in api.cpp.
// ---------------------------------------------------------------------------
template <int BITS, bool SB_BF16, int MT, int R>
static hipError_t launch_qmv_t(const QmvArgs& a, int grid, size_t lds) {
  auto kern = qmv_kernel<BITS, SB_BF16, MT, R>;
  if (lds > 65536) {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, a.stream, a.x, a.w, a.s, a.b, a.y,
                     static_cast<int>(a.N), static_cast<int>(a.K), a.glog2, a.x_vec);
  return hipGetLastError();
}

template <int BITS, bool SB_BF16, int R>
static hipError_t launch_qmv_mt(const QmvArgs& a, int mt, int grid, size_t lds) {
  switch (mt) {
    case 1: return launch_qmv_t<BITS, SB_BF16, 1, R>(a, grid, lds);
    case 2: return launch_qmv_t<BITS, SB_BF16, 2, R>(a, grid, lds);
    case 3: return launch_qmv_t<BITS, SB_BF16, 3, R>(a, grid, lds);
    case 4: return launch_qmv_t<BITS, SB_BF16, 4, R>(a, grid, lds);
    case 5: return launch_qmv_t<BITS, SB_BF16, 5, R>(a, grid, lds);
    case 6: return launch_qmv_t<BITS, SB_BF16, 6, R>(a, grid, lds);
    case 7: return launch_qmv_t<BITS, SB_BF16, 7, R>(a, grid, lds);
    default: return launch_qmv_t<BITS, SB_BF16, 8, R>(a, grid, lds);
  }
}

template <int BITS, bool SB_BF16>
static hipError_t launch_qmv_bits(const QmvArgs& a, int mt, int R, int grid, size_t lds) {
  // R * MT live outputs per lane are capped at 32.
  if (R == 4 && mt <= 8) return launch_qmv_mt<BITS, SB_BF16, 4>(a, mt, grid, lds);
  if (R == 2) return launch_qmv_mt<BITS, SB_BF16, 2>(a, mt, grid, lds);
  return launch_qmv_mt<BITS, SB_BF16, 1>(a, mt, grid, lds);
}

size_t qmv_lds_need(int bits, int mt, int64_t K) {
  return bits == 4 ? qmv_lds_bytes<4>(mt, static_cast<int>(K))
                   : qmv_lds_bytes<8>(mt, static_cast<int>(K));
}

int qmv_pick_rows(const DeviceInfo& dev, int64_t N, int mt) {
  const int64_t target = static_cast<int64_t>(dev.num_cu) * 8;  // waves to fill the chip
  int R = 1;
  if ((N + 3) / 4 >= target) R = 4;
  else if ((N + 1) / 2 >= target) R = 2;
  while (R > 1 && R * mt > 16) R /= 2;  // bound live accumulators and LDS reads
  return R;
}

QmvPlan qmv_plan(const DeviceInfo& dev, int64_t N, int64_t K, int bits, int mt, int rows_override) {
  QmvPlan p{};
  p.mt = mt;
  p.rows = rows_override > 0 ? rows_override : qmv_pick_rows(dev, N, mt);
  p.lds = qmv_lds_need(bits, mt, K);
  const int64_t nrb = (N + p.rows - 1) / p.rows;
  const int64_t blocks_needed = (nrb + 3) / 4;
  int per_cu = static_cast<int>(dev.lds_per_cu / (p.lds > 0 ? p.lds : 1));
  per_cu = per_cu < 1 ? 1 : (per_cu > 8 ? 8 : per_cu);
  const int64_t cap = static_cast<int64_t>(dev.num_cu) * per_cu;
  p.grid = static_cast<int>(blocks_needed < cap ? blocks_needed : cap);
  return p;
}

hipError_t launch_qmv_slice(const QmvArgs& a, const DeviceInfo& dev, int mt) {
  const QmvPlan p = qmv_plan(dev, a.N, a.K, a.bits, mt, a.rows_per_wave);
  const int R = p.rows, grid = p.grid;
  const size_t lds = p.lds;
  if (a.bits == 4)
    return a.sb_bf16 ? launch_qmv_bits<4, true>(a, mt, R, grid, lds)
                     : launch_qmv_bits<4, false>(a, mt, R, grid, lds);
  return a.sb_bf16 ? launch_qmv_bits<8, true>(a, mt, R, grid, lds)
                   : launch_qmv_bits<8, false>(a, mt, R, grid, lds);
}

}  // namespace mxq
