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
//  * Codes go under an f16 exponent (two per v_and_or_b32) and meet the
//    activations in v_dot2_f32_f16 with f32 accumulation.  8-bit codes are
//    exact integers (1024 + c, less 1024); 4-bit codes keep a power-of-two
//    offset (64 + c, f16; 128 + c, bf16) that the bias factor removes.  A
//    segment never straddles a group (group_size >= 32 codes), so its scale and
//    bias are applied once per segment in f32:
//        acc += s * sum(x*q) + b * sum(x)     (zero-point form, mlxcel #574
//                                              "Upstream status refresh")
//    where sum(x) over the segment is precomputed; with an offset E on the
//    codes, sum(x*(E + q)) = sum(x*q) + E*sum(x) and b becomes b - E*s.
//  * x is staged once per workgroup in LDS, already reordered into the pair
//    order of the unpack, laid out [m][chunk][segment] so that the 64 lanes'
//    16-byte reads hit consecutive addresses (no bank conflicts), together
//    with the per-segment sums of x.
//  * Partial sums of the R*M outputs are reduced across the wave with a
//    "transpose" butterfly: each cross-lane exchange stage halves the number
//    of live values per lane (R*M - 1 exchanges instead of 6*R*M), after which
//    each value's partial sums lie in an aligned group of 64/(R*M) lanes and
//    are summed with DPP row moves (no LDS round trips, which dominate the
//    latency of the small launches).  Everything is in a fixed order: results
//    are deterministic.
//  * The kernel argument holds one 64-byte record per problem of a grouped
//    launch; a workgroup finds its problem from the block ranges with scalar
//    selects and fetches the record with one scalar load.  The first
//    problem's record is read with the block ranges, so single-problem
//    launches wait for one scalar round trip before the first weight load.
//  * Workgroups are persistent (grid-stride over row blocks) so the x staging
//    is paid once per workgroup, not once per row block.
#include <climits>
#include <map>
#include <mutex>
#include <tuple>

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
         (SegTraits<BITS>::kChunksPerSeg * 16 + 4) + static_cast<size_t>(MT) * 4;  // + int8 mode's row maxima
}

constexpr int kQmvBlock = 256;  // threads per workgroup (the host always launches this many)

// Sum of v over each aligned group of L lanes (L a power of two <= 64), left
// in the group's last lane (for L <= 16 in every lane of the group), through
// DPP moves: two quad swaps, the half-row and row mirrors, then the row
// broadcasts of lane 15 into the next row and of lane 31 into rows 2 and 3
// (rows the broadcast does not write add zero).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float u) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(u), CTRL, ROW_MASK, 0xF, false));
}
template <int L>
__device__ __forceinline__ float group_sum_to_last(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1, 0xF>(v);   // quad_perm 1,0,3,2
  if constexpr (L >= 4) v += dpp_f32<0x4E, 0xF>(v);   // quad_perm 2,3,0,1
  if constexpr (L >= 8) v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_f32<0x140, 0xF>(v); // row_mirror
  if constexpr (L >= 32) v += dpp_f32<0x142, 0xA>(v); // row_bcast:15 into rows 1 and 3
  if constexpr (L >= 64) v += dpp_f32<0x143, 0xC>(v); // row_bcast:31 into rows 2 and 3
  return v;
}

// Loads of one work item: R rows x one 16-byte segment, plus their scales and biases.
template <int R>
struct QmvItem {
  u4 w[R];
  uint16_t s[R], b[R];
  uint16_t ob;  // output bias of the row this lane stores (when there is one)
};

// Activation pair order of the unpack for one 16-byte chunk (8 activations):
// 4-bit codes pair (c0, c4) (c1, c5) ..., f16 8-bit codes (c0, c2) (c1, c3),
// bf16 8-bit codes in natural order.
template <int BITS, bool XB>
__device__ __forceinline__ u4 perm_x(u4 v) {
  if constexpr (BITS == 4) {
    return perm_x_w4(v);
  } else if constexpr (XB) {
    return v;
  } else {
    return perm_x_w8(v);
  }
}

// Activation modes of the decode kernel.
constexpr int kActF16 = 0;   // x, y f16
constexpr int kActBF16 = 1;  // x, y bf16
constexpr int kActI8 = 2;    // x f16, quantized per row to int8 inside the kernel; y f16

// Largest value over the wave (non-negative inputs), in every lane: DPP moves
// fold it into lane 63, which is then read as a wave-uniform value.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xF>(v));
  v = fmaxf(v, dpp_f32<0x4E, 0xF>(v));
  v = fmaxf(v, dpp_f32<0x141, 0xF>(v));
  v = fmaxf(v, dpp_f32<0x140, 0xF>(v));
  v = fmaxf(v, dpp_f32<0x142, 0xA>(v));
  v = fmaxf(v, dpp_f32<0x143, 0xC>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ACT: activation mode (kActF16, kActBF16, kActI8).
template <int BITS, bool SB_BF16, int MT, int R, bool XD, int ACT>
__global__ __launch_bounds__(kQmvBlock) void qmv_kernel(const QmvBatch batch) {
  constexpr bool XB = ACT == kActBF16;
  constexpr bool XI = ACT == kActI8;
  // This workgroup's problem: the number of problems whose block range ends
  // at or before this block.  The block ranges, problem 0's record and the
  // group size are read in one batch of scalar loads (an empty asm use of all
  // of them keeps the compiler from spreading them over several round trips);
  // blocks of the other problems then fetch their record with one more.
  QmvSlot pb = batch.first;
  const int glog2 = batch.glog2;
  int ends[kMaxGroup - 1];
#pragma unroll
  for (int i = 0; i + 1 < kMaxGroup; ++i) ends[i] = batch.block_end[i];
  asm volatile("" ::"s"(pb.x), "s"(pb.w), "s"(pb.s), "s"(pb.b), "s"(pb.y), "s"(pb.ob), "s"(pb.N), "s"(pb.K),
               "s"(pb.block_begin), "s"(pb.nblk), "s"(glog2), "s"(ends[0]), "s"(ends[1]), "s"(ends[2]),
               "s"(ends[3]), "s"(ends[4]), "s"(ends[5]), "s"(ends[6]), "s"(ends[7]), "s"(ends[8]), "s"(ends[9]),
               "s"(ends[10]), "s"(ends[11]), "s"(ends[12]), "s"(ends[13]), "s"(ends[14]));
  int p = 0;
#pragma unroll
  for (int i = 0; i + 1 < kMaxGroup; ++i) p = static_cast<int>(blockIdx.x) >= ends[i] ? i + 1 : p;
  if (p != 0) pb = batch.rest[p - 1];
  const int blk = static_cast<int>(blockIdx.x) - pb.block_begin;
  const int nblk = pb.nblk;
  const uint16_t* __restrict__ x = pb.x;
  const uint32_t* __restrict__ W = pb.w;
  const uint16_t* __restrict__ S = pb.s;
  const uint16_t* __restrict__ B = pb.b;
  uint16_t* __restrict__ y = pb.y;
  const uint16_t* __restrict__ ob = pb.ob;
  const bool has_ob = ob != nullptr;
  const int N = pb.N, K = pb.K;
  const bool x_vec = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  constexpr int CPS = SegTraits<BITS>::kChunksPerSeg;
  constexpr int CODES = SegTraits<BITS>::kCodesPerSeg;
  constexpr int NP = (BITS == 4) ? 16 : 8;  // f16 code pairs per segment
  constexpr int V = R * MT;
  constexpr int VP = V <= 1 ? 1 : V <= 2 ? 2 : V <= 4 ? 4 : V <= 8 ? 8 : V <= 16 ? 16 : 32;
  static_assert(V <= 32, "too many live outputs per lane");

  extern __shared__ __align__(16) unsigned char smem[];
  const int nseg = K * BITS / 128;   // segments per row
  const int kw = K * BITS / 32;      // words per row
  const int G = K >> glog2;          // groups per row
  u4* xs = reinterpret_cast<u4*>(smem);                                     // [MT][CPS][nseg]
  float* xsum = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * CPS * nseg * 16);  // [MT][nseg]

  const int lane = threadIdx.x & (kWave - 1);
  // Output this lane stores after the wave reduction (see the butterfly in
  // step): its value index, and from it the row offset within a row block.
  int my_idx = 0;
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int live = VP >> s;
    if (live >= 2 && (lane & (32 >> s))) my_idx += live / 2;
  }
  const int my_r = min(my_idx, V - 1) / MT;
  // wave-uniform values live in scalar registers: all row addressing is scalar
  // (64-bit row bases), and each load adds one 32-bit per-lane offset within
  // the row to its row's base
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int waves_per_block = kQmvBlock / kWave;
  const int nrb = (N + R - 1) / R;
  const int jn = (nseg + kWave - 1) / kWave;
  const int stride = nblk * waves_per_block;
  const uint32_t wrow_bytes = static_cast<uint32_t>(kw) * 4u;
  const uint32_t sbrow_bytes = static_cast<uint32_t>(G) * 2u;
  const char* Wb = reinterpret_cast<const char*>(W);
  const char* Sb = reinterpret_cast<const char*>(S);
  const char* Bb = reinterpret_cast<const char*>(B);

  // Loads are unconditional and branch-free (indices clamped into range) so the
  // compiler's load counters stay exact: a conditional load would make it wait
  // for every outstanding load, including the prefetched ones.  Past a wave's
  // last item the loads are dummies aimed at the activation row (a few KiB,
  // cache-resident) by a wave-uniform select of the base pointers: with row 0
  // every offset ends within K*BITS/8 <= 2*K bytes, the row's size, and the
  // 16-byte loads start from x rounded down to 16 bytes (same page as x).
  const char* Xb = reinterpret_cast<const char*>(x);
  const char* Xw = Xb - (reinterpret_cast<uintptr_t>(x) & 15u);
  auto load_item = [&](QmvItem<R>& it, int rbl, int jl, bool dummy) {
    const int seg = min(lane + jl * kWave, nseg - 1);
    const uint32_t wl = static_cast<uint32_t>(seg) * 16u;
    const uint32_t sl = static_cast<uint32_t>((seg * CODES) >> glog2) * 2u;
    const char* wbase = dummy ? Xw : Wb;
    const char* sbase = dummy ? Xb : Sb;
    const char* bbase = dummy ? Xb : Bb;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = dummy ? 0u : static_cast<uint32_t>(min(rbl * R + r, N - 1));  // tail rows re-read the last row; never stored
      // the row's base address is a wave-uniform 64-bit value (W may exceed
      // 4 GiB); the lane adds its 32-bit offset within the row
      // (the empty asm keeps the global row bases in SGPRs, so each load takes
      // the SGPR-base + 32-bit lane-offset form instead of a 64-bit lane address)
      gptr<const char> wrow = to_global(wbase + static_cast<size_t>(row) * wrow_bytes);
      gptr<const char> srow = to_global(sbase + static_cast<size_t>(row) * sbrow_bytes);
      gptr<const char> brow = to_global(bbase + static_cast<size_t>(row) * sbrow_bytes);
      asm volatile("" : "+s"(wrow), "+s"(srow), "+s"(brow));
      // W, scales and biases are each read exactly once: non-temporal loads keep
      // them from displacing reusable lines (measured ~7% faster on lm_head)
      it.w[r] = __builtin_nontemporal_load(reinterpret_cast<gptr<const u4>>(wrow + wl));
      it.s[r] = __builtin_nontemporal_load(reinterpret_cast<gptr<const uint16_t>>(srow + sl));
      it.b[r] = __builtin_nontemporal_load(reinterpret_cast<gptr<const uint16_t>>(brow + sl));
    }
    // the stored row's output bias, fetched with every item of the row block
    // (so the one the block ends with has it); without a bias, a harmless
    // read of x[0] whose value is never used
    const uint32_t orow = dummy ? 0u : static_cast<uint32_t>(min(rbl * R + my_r, N - 1));
    it.ob = *reinterpret_cast<const uint16_t*>(has_ob ? reinterpret_cast<const char*>(ob) + orow * 2u : Xb);
  };

  // The first item's loads go out before the x staging, to overlap the two.
  int rb = blk * waves_per_block + wave;
  int j = 0;
  QmvItem<R> cur;
  load_item(cur, min(rb, nrb - 1), 0, false);

  // ---- activations -------------------------------------------------------
  // XD (a row fits in one segment step, M <= 2): each lane's segment of x is
  // the same for the whole kernel, so it goes straight into registers with the
  // first weight loads -- no LDS, no barrier.  Otherwise x is staged once per
  // workgroup in LDS, reordered, with its per-segment sums.
  auto load_x_global = [&](int m, int seg, u4 (&v)[CPS]) {
    const uint16_t* xp = x + static_cast<size_t>(m) * K + seg * CODES;
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      if (x_vec) {
        v[c] = *reinterpret_cast<const u4*>(xp + 8 * c);
      } else {
        uint32_t t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          t[i] = static_cast<uint32_t>(xp[8 * c + 2 * i]) |
                 (static_cast<uint32_t>(xp[8 * c + 2 * i + 1]) << 16);
        v[c] = u4{t[0], t[1], t[2], t[3]};
      }
    }
  };
  constexpr int NPX = (BITS == 4) ? 16 : 8;
  uint32_t xreg[XD ? MT : 1][NPX];
  float xsreg[XD ? MT : 1];
  // int8 mode: per-row scale sx = amax / 127 and factor r = 127 / amax (both
  // f32 quotients; a zero row gives r = 0, sx = 0, so its codes are 0)
  float sxm[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) sxm[m] = 1.0f;
  auto row_scales = [&](float amax, float& r, float& sx) {
    const bool z = !(amax > 0.0f);
    r = z ? 0.0f : 127.0f / amax;
    sx = z ? 0.0f : amax / 127.0f;
  };
  if constexpr (XD) {
    const int seg = min(lane, nseg - 1);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u4 v[CPS];
      load_x_global(m, seg, v);
      if constexpr (XI) {
        // the row lies within this wave's lanes (one segment step), so the
        // wave finds its largest |x| itself
        float am = 0.0f;
#pragma unroll
        for (int c = 0; c < CPS; ++c) am = fmaxf(am, absmax8_f16(v[c]));
        float r;
        row_scales(wave_max_nonneg(am), r, sxm[m]);
        int sum = 0;
#pragma unroll
        for (int c = 0; c < CPS; ++c) quant_chunk_i8<BITS>(v[c], r, xreg[m][2 * c], xreg[m][2 * c + 1], sum);
        xsreg[m] = static_cast<float>(sum);
      } else {
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < CPS; ++c) {
          sum += sum8_act<XB>(v[c]);
          const u4 p = perm_x<BITS, XB>(v[c]);
          xreg[m][4 * c] = p.x;
          xreg[m][4 * c + 1] = p.y;
          xreg[m][4 * c + 2] = p.z;
          xreg[m][4 * c + 3] = p.w;
        }
        xsreg[m] = sum;
      }
    }
    if (rb >= nrb) return;
  } else if constexpr (XI) {
    // int8 mode, staged: pass 1 finds each row's largest |x| (LDS atomic max
    // on the f32 bits, which order like unsigned integers for values >= 0),
    // pass 2 quantizes into LDS with the row's factor
    uint32_t* amax_s = reinterpret_cast<uint32_t*>(xsum + MT * nseg);
    if (threadIdx.x < MT) amax_s[threadIdx.x] = 0u;
    __syncthreads();
    for (int u = threadIdx.x; u < MT * nseg; u += kQmvBlock) {
      const int m = u / nseg;
      const int seg = u - m * nseg;
      u4 v[CPS];
      load_x_global(m, seg, v);
      float am = 0.0f;
#pragma unroll
      for (int c = 0; c < CPS; ++c) am = fmaxf(am, absmax8_f16(v[c]));
      atomicMax(&amax_s[m], __float_as_uint(am));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float r;
      row_scales(__uint_as_float(amax_s[m]), r, sxm[m]);
    }
    for (int u = threadIdx.x; u < MT * nseg; u += kQmvBlock) {
      const int m = u / nseg;
      const int seg = u - m * nseg;
      float r, sx;
      row_scales(__uint_as_float(amax_s[m]), r, sx);
      u4 v[CPS];
      load_x_global(m, seg, v);
      int sum = 0;
      uint32_t d[2 * CPS];
#pragma unroll
      for (int c = 0; c < CPS; ++c) quant_chunk_i8<BITS>(v[c], r, d[2 * c], d[2 * c + 1], sum);
#pragma unroll
      for (int c = 0; c < CPS / 2; ++c)
        xs[(m * CPS + c) * nseg + seg] = u4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
      xsum[m * nseg + seg] = static_cast<float>(sum);
    }
    __syncthreads();
    if (rb >= nrb) return;  // no block-level barrier follows
  } else {
    for (int u = threadIdx.x; u < MT * nseg; u += kQmvBlock) {
      const int m = u / nseg;
      const int seg = u - m * nseg;
      u4 v[CPS];
      load_x_global(m, seg, v);
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        sum += sum8_act<XB>(v[c]);
        xs[(m * CPS + c) * nseg + seg] = perm_x<BITS, XB>(v[c]);
      }
      xsum[m * nseg + seg] = sum;
    }
    __syncthreads();
    if (rb >= nrb) return;  // no block-level barrier follows
  }

  const uint32_t magic = XB ? kMagicB : BITS == 4 ? kMagic64 : kMagic;
  // the per-segment bias factor: b, or b - 128 s when the codes carry +128
  // (bf16 4-bit), b - 64 s when they carry +64 (f16 4-bit), or b + 128 s when
  // they carry -128 (int8 mode, 8-bit codes as signed bytes c - 128); the
  // offsets are powers of two, so the factor is exact in f32 whenever b and
  // the multiple of s lie within 2^13 of each other in magnitude
  auto bias_term = [&](uint16_t bbits, float sc) {
    const float b = sb_to_f32<SB_BF16>(bbits);
    if constexpr (XB && BITS == 4) {
      return __builtin_fmaf(-128.0f, sc, b);
    } else if constexpr (!XI && BITS == 4) {
      return __builtin_fmaf(-64.0f, sc, b);
    } else if constexpr (XI && BITS == 8) {
      return __builtin_fmaf(128.0f, sc, b);
    } else {
      return b;
    }
  };
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  // segment dot product of one row's codes with one activation row's pairs
  // (4-bit codes carry +128 (bf16) or +64 (f16) each; the bias term takes the
  // offset times sum(x) back)
  auto seg_dot = [&](const uint32_t (&q)[NP], const uint32_t (&xp)[NP]) {
    if constexpr (XI) {
      // int8 codes against int8 activations, four products per v_dot4, exact
      constexpr int NQ = 2 * CPS;
      int d0 = 0, d1 = 0;
#pragma unroll
      for (int p = 0; p < NQ; p += 2) {
        d0 = __builtin_amdgcn_sdot4(static_cast<int>(q[p]), static_cast<int>(xp[p]), d0, false);
        d1 = __builtin_amdgcn_sdot4(static_cast<int>(q[p + 1]), static_cast<int>(xp[p + 1]), d1, false);
      }
      return static_cast<float>(d0 + d1);
    } else if constexpr (XB) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; p += 2) {
        d0 = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q[p]), as_b2(xp[p]), d0, false);
        d1 = __builtin_amdgcn_fdot2_f32_bf16(as_b2(q[p + 1]), as_b2(xp[p + 1]), d1, false);
      }
      return d0 + d1;
    } else if constexpr (BITS == 4) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; p += 2) {
        d0 = __builtin_amdgcn_fdot2(as_h2(q[p]), as_h2(xp[p]), d0, false);
        d1 = __builtin_amdgcn_fdot2(as_h2(q[p + 1]), as_h2(xp[p + 1]), d1, false);
      }
      return d0 + d1;
    } else {
      float d = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) d = __builtin_amdgcn_fdot2(as_h2(q[p]), as_h2(xp[p]), d, false);
      return d;
    }
  };
  auto unpack_row = [&](const u4& wv, uint32_t (&q)[NP]) {
    const uint32_t wr[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XI && BITS == 4) {
        // nibbles to bytes: even codes (0, 2, 4, 6) and odd codes (1, 3, 5, 7)
        q[2 * i] = wr[i] & 0x0F0F0F0Fu;
        q[2 * i + 1] = (wr[i] >> 4) & 0x0F0F0F0Fu;
      } else if constexpr (XI) {
        q[i] = wr[i] ^ 0x80808080u;  // c - 128 as a signed byte
      } else if constexpr (XB && BITS == 4) {
        uint32_t t[4];
        unpack_w4_off(wr[i], magic, t);
#pragma unroll
        for (int p = 0; p < 4; ++p) q[4 * i + p] = t[p];
      } else if constexpr (XB) {
        uint32_t t[2];
        unpack_w8_bf16(wr[i], t);
        q[2 * i] = t[0];
        q[2 * i + 1] = t[1];
      } else if constexpr (BITS == 4) {
        uint32_t t[4];
        unpack_w4_off64(wr[i], magic, t);
#pragma unroll
        for (int p = 0; p < 4; ++p) q[4 * i + p] = t[p];
      } else {
        h2 t[2];
        unpack_w8_ao(wr[i], magic, t);
        q[2 * i] = as_u32(t[0]);
        q[2 * i + 1] = as_u32(t[1]);
      }
    }
  };
  auto load_x = [&](int m, int seg, uint32_t (&xp)[NP]) {
    if constexpr (XD) {
#pragma unroll
      for (int p = 0; p < NP; ++p) xp[p] = xreg[m][p];
      return;
    }
    constexpr int XC = XI ? CPS / 2 : CPS;  // 16-byte chunks of one segment's activations
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const u4 xv = xs[(m * CPS + c) * nseg + seg];
      xp[4 * c] = xv.x;
      xp[4 * c + 1] = xv.y;
      xp[4 * c + 2] = xv.z;
      xp[4 * c + 3] = xv.w;
    }
  };

  // Compute one item (row block rbl, segment step jl); when it completes the
  // row block, reduce the partial sums across the wave and store them.
  auto step = [&](const QmvItem<R>& it, int rbl, int jl, bool block_done) {
    // Branch-free: lanes past the end of the row (ragged last step) compute on a
    // clamped, valid segment and discard the result with a select, so every
    // path consumes the loads (keeping the compiler's load counters exact).
    const int seg_raw = lane + jl * kWave;
    const bool active = seg_raw < nseg;
    const int seg = min(seg_raw, nseg - 1);
    if constexpr (MT <= 2) {
      // few activation rows: keep them in registers, unpack one W row at a time
      uint32_t xp[MT][NP];
      float xsm[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        load_x(m, seg, xp[m]);
        xsm[m] = XD ? xsreg[m] : xsum[m * nseg + seg];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t q[NP];
        unpack_row(it.w[r], q);
        const float sc = sb_to_f32<SB_BF16>(it.s[r]);
        const float bi = bias_term(it.b[r], sc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float t = __builtin_fmaf(bi, xsm[m], __builtin_fmaf(sc, seg_dot(q, xp[m]), acc[r][m]));
          acc[r][m] = active ? t : acc[r][m];
        }
      }
    } else {
      // many activation rows: unpack all R rows once, stream x rows from LDS
      uint32_t q[R][NP];
#pragma unroll
      for (int r = 0; r < R; ++r) unpack_row(it.w[r], q[r]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint32_t xp[NP];
        load_x(m, seg, xp);
        const float xsm = XD ? xsreg[XD ? m : 0] : xsum[m * nseg + seg];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float sc = sb_to_f32<SB_BF16>(it.s[r]);
          const float t = __builtin_fmaf(bias_term(it.b[r], sc), xsm, __builtin_fmaf(sc, seg_dot(q[r], xp), acc[r][m]));
          acc[r][m] = active ? t : acc[r][m];
        }
      }
    }
    if (!block_done) return;

    // ---- transpose butterfly over the 64 lanes -------------------------
    // While several values are live per lane, each stage swaps halves with
    // the lane `off` away; then each value's partial sums sit in an aligned
    // group of kLow lanes and are summed within the group with DPP moves.
    float v[VP];
#pragma unroll
    for (int i = 0; i < VP; ++i) v[i] = (i < V) ? acc[i / MT][i % MT] * (XI ? sxm[i % MT] : 1.0f) : 0.0f;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      const int off = 32 >> s;
      const int live = VP >> s;  // values still live per lane before this stage
      if (live >= 2) {
        const int h = live / 2;
        if (off >= 16) {
          // gfx950's lane swaps do the exchange in one VALU op per pair, no
          // LDS crossbar and no selects: v_permlane32_swap trades the upper
          // half of v[i] for the lower half of v[i + h] (v_permlane16_swap:
          // the odd 16-lane rows for the even ones), so that v[i] + v[i + h]
          // afterwards is the sum with the partner lane `off` away of v[i] in
          // the lanes with bit `off` clear and of v[i + h] in the others
#pragma unroll
          for (int i = 0; i < h; ++i) {
            const auto sw = off == 32
                                ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + h]), false, false)
                                : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + h]), false, false);
            v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          }
        } else {
          const bool upper = (lane & off) != 0;
#pragma unroll
          for (int i = 0; i < h; ++i) {
            const float send = upper ? v[i] : v[i + h];
            const float keep = upper ? v[i + h] : v[i];
            v[i] = keep + __shfl_xor(send, off, kWave);
          }
        }
      }
    }
    constexpr int kLow = kWave / VP;  // lanes sharing one value index
    v[0] = group_sum_to_last<kLow>(v[0]);
    // the group's last lane holds the total; its value index is the sum over
    // the exchange stages of bit(lane, off) * h (bits above the group)
    if ((lane & (kLow - 1)) == kLow - 1) {
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
        const int row = rbl * R + r;
        const float o = has_ob ? sb_to_f32<XB>(it.ob) : 0.0f;
        if (row < N) y[static_cast<size_t>(m) * N + row] = f32_to_act_bits<XB>(v[0] + o);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
  };

  // A ring of item buffers: while an item is computed, the loads of the next
  // NBUF - 1 items are in flight, and no register copy of in-flight data is
  // ever made (a copy would force a wait for those loads).  Loads are never
  // conditional: loads past a wave's last item are dummies of load_item, which
  // keeps the compiler's load counters exact.  The loop has a single exit:
  // with two exits the compiler's wait analysis merges them into the loop
  // header and makes every iteration wait for the prefetch.
  // Items in flight per wave: two at four rows per item (the large class,
  // which runs as many workgroups as fit instead; a third item there measured
  // 2-3 % slower), three otherwise (the mid and small classes: each wave has
  // only a few items, and the third hides more of each item's compute behind
  // the loads -- gate+up 6.4 -> 6.0 us, down 5.5 -> 5.2 us; a fourth measured
  // slower, gate+up 6.5 us).
  constexpr int NBUF = R == 4 ? 2 : 3;
  auto advance = [&](int& rbv, int& jv) {
    if (++jv == jn) {
      jv = 0;
      rbv += stride;
    }
  };
  const int n_items = ((nrb - 1 - rb) / stride + 1) * jn;  // this wave's items, >= 1
  // A ring of NBUF item buffers: buffer k holds item i + k at the top of a
  // trip; each step first issues the loads of item i + k + NBUF - 1 into the
  // buffer the previous trip's last step freed, then computes item i + k.
  QmvItem<R> buf[NBUF];
  int prb[NBUF], pj[NBUF];  // (row block, segment step) of the item in each buffer
  buf[0] = cur;
  prb[0] = rb;
  pj[0] = j;
#pragma unroll
  for (int k = 1; k < NBUF - 1; ++k) {
    prb[k] = prb[k - 1];
    pj[k] = pj[k - 1];
    advance(prb[k], pj[k]);
    load_item(buf[k], prb[k], pj[k], k >= n_items);  // a dummy past the end
  }
  int i = 0;  // the item in buf[0]
  for (; i + NBUF - 1 < n_items; i += NBUF) {
#pragma unroll
    for (int k = 0; k < NBUF; ++k) {
      const int kl = (k + NBUF - 1) % NBUF, kp = (k + NBUF - 2) % NBUF;
      prb[kl] = prb[kp];
      pj[kl] = pj[kp];
      advance(prb[kl], pj[kl]);  // item i + k + NBUF - 1
      load_item(buf[kl], prb[kl], pj[kl], i + k + NBUF - 1 >= n_items);
      __builtin_amdgcn_sched_barrier(0);  // keep the whole load block ahead of the compute
      step(buf[k], prb[k], pj[k], pj[(k + 1) % NBUF] == 0);
    }
  }
  // fewer than NBUF items left, in buf[0 .. NBUF - 2]; the last ends its row block
#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (i + k < n_items) step(buf[k], prb[k], pj[k], i + k + 1 >= n_items || pj[(k + 1) % NBUF] == 0);
}

// ---------------------------------------------------------------------------
// Host side: instantiation table, occupancy-sized persistent grid, launch.
// Validation happens in api.cpp before any of this runs.
// ---------------------------------------------------------------------------
namespace {

template <int BITS, bool SB_BF16, int R, int ACT>
const void* qmv_ptr_mt(int mt, bool xd) {
  if (xd) {
    if (mt == 1) return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 1, R, true, ACT>);
    return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 2, R, true, ACT>);
  }
  switch (mt) {
    case 1: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 1, R, false, ACT>);
    case 2: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 2, R, false, ACT>);
    case 3: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 3, R, false, ACT>);
    case 4: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 4, R, false, ACT>);
    case 5: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 5, R, false, ACT>);
    case 6: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 6, R, false, ACT>);
    case 7: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 7, R, false, ACT>);
    default: return reinterpret_cast<const void*>(&qmv_kernel<BITS, SB_BF16, 8, R, false, ACT>);
  }
}

template <int BITS, bool SB_BF16, int ACT>
const void* qmv_ptr_r(int mt, int R, bool xd) {
  if (R == 4) return qmv_ptr_mt<BITS, SB_BF16, 4, ACT>(mt, xd);
  if (R == 2) return qmv_ptr_mt<BITS, SB_BF16, 2, ACT>(mt, xd);
  return qmv_ptr_mt<BITS, SB_BF16, 1, ACT>(mt, xd);
}

template <int ACT>
const void* qmv_ptr_x(int bits, bool bf16, int mt, int R, bool xd) {
  if (bits == 4) return bf16 ? qmv_ptr_r<4, true, ACT>(mt, R, xd) : qmv_ptr_r<4, false, ACT>(mt, R, xd);
  return bf16 ? qmv_ptr_r<8, true, ACT>(mt, R, xd) : qmv_ptr_r<8, false, ACT>(mt, R, xd);
}

const void* qmv_kernel_ptr(int bits, bool bf16, int act, int mt, int R, bool xd) {
  if (act == kActI8) return qmv_ptr_x<kActI8>(bits, bf16, mt, R, xd);
  return act == kActBF16 ? qmv_ptr_x<kActBF16>(bits, bf16, mt, R, xd) : qmv_ptr_x<kActF16>(bits, bf16, mt, R, xd);
}

// Rows of W per wave step and the grid, by size class of N (measured on
// MI355X with a read probe and traced launch-shape sweeps):
//  * large (N >= 64 rows per CU, e.g. a vocabulary projection): R = 4 rows
//    of one 16-byte segment per lane (R = 2 when a row spans several segment
//    steps), as many workgroups of 4 waves per CU as fit (5 at 94 VGPRs), each
//    wave holding two items in flight (a third measured slower at every
//    workgroup count);
//  * mid (N >= 16 rows per CU): R = 2, 2 workgroups per CU (fewer, longer
//    waves beat one row per wave by ~15 %; R = 4 measured the same);
//  * small: one row per wave step; as many waves as the rows allow when x is
//    staged in LDS, one workgroup per CU when x sits in registers (below);
//    such launches are dominated by their fixed cost (~3-4 us on this part).
enum class SizeClass { kSmall, kMid, kLarge };

SizeClass qmv_class(const DeviceInfo& dev, int64_t N) {
  if (N >= static_cast<int64_t>(dev.num_cu) * 64) return SizeClass::kLarge;
  if (N >= static_cast<int64_t>(dev.num_cu) * 16) return SizeClass::kMid;
  return SizeClass::kSmall;
}

int qmv_pick_rows(const DeviceInfo& dev, int64_t N, int64_t K, int bits, int mt) {
  int rows = 1;
  const SizeClass c = qmv_class(dev, N);
  if (c == SizeClass::kLarge) rows = (K * bits / 128 <= kWave) ? 4 : 2;
  if (c == SizeClass::kMid) rows = 2;
  while (rows > 1 && rows * mt > 16) rows /= 2;  // bound live accumulators and registers
  return rows;
}

// Small launches with the activations in registers take one workgroup per CU
// per problem, so that a wave holds two or more items and the item pipeline
// has something to overlap (q+k+v: 3.92 -> 3.65 us); with x staged in LDS once
// per workgroup (long K) more workgroups stay faster (down: 5.11 against 5.72
// us at one per CU).
int qmv_blocks_per_cu_cap(const DeviceInfo& dev, int64_t N, int occ, bool xd) {
  switch (qmv_class(dev, N)) {
    case SizeClass::kLarge: return occ;  // as many as fit: lm_head 24.9 / 24.3 / 24.2 / 23.9 us at 2 / 3 / 4 / 5
    case SizeClass::kMid: return occ < 2 ? occ : 2;
    default: return xd ? (occ < 1 ? occ : 1) : occ;
  }
}

std::mutex g_occ_mu;
std::map<std::tuple<int, const void*, size_t>, int> g_occ;  // (device, kernel, lds) -> blocks/CU

int blocks_per_cu(const DeviceInfo& dev, const void* kern, size_t lds) {
  const auto key = std::make_tuple(dev.device, kern, lds);
  {
    std::lock_guard<std::mutex> lk(g_occ_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) return it->second;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kQmvBlock, lds) != hipSuccess || nb < 1) {
    (void)hipGetLastError();
    nb = 1;
  }
  std::lock_guard<std::mutex> lk(g_occ_mu);
  g_occ[key] = nb;
  return nb;
}

}  // namespace

size_t qmv_lds_need(int bits, int mt, int64_t K) {
  return bits == 4 ? qmv_lds_bytes<4>(mt, static_cast<int>(K))
                   : qmv_lds_bytes<8>(mt, static_cast<int>(K));
}

// One instantiation serves every problem of a group: R from the problem with
// the most rows, activations in registers only if every row fits in one
// segment step, LDS sized for the largest K.  Each problem gets its own block
// range, sized as it would be alone.
QmvPlan qmv_plan_group(const DeviceInfo& dev, const int64_t* Ns, const int64_t* Ks, int count, int bits,
                       bool sb_bf16, int act, int mt, int* grids) {
  QmvPlan p{};
  p.mt = mt;
  int big = 0;
  bool xd = mt <= 2;
  size_t lds = 0;
  for (int i = 0; i < count; ++i) {
    if (Ns[i] > Ns[big]) big = i;
    xd = xd && (Ks[i] * bits / 128 <= kWave);
    const size_t l = qmv_lds_need(bits, mt, Ks[i]);
    lds = l > lds ? l : lds;
  }
  p.rows = qmv_pick_rows(dev, Ns[big], Ks[big], bits, mt);
  p.xdirect = xd;
  p.lds = xd ? 0 : lds;
  p.kernel = qmv_kernel_ptr(bits, sb_bf16, act, mt, p.rows, p.xdirect);
  if (p.lds > 65536 && ensure_dynamic_lds(p.kernel, p.lds) != hipSuccess) (void)hipGetLastError();
  const int occ = blocks_per_cu(dev, p.kernel, p.lds);
  p.grid = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t nrb = (Ns[i] + p.rows - 1) / p.rows;
    const int64_t blocks_needed = (nrb + 3) / 4;
    const int per_cu = qmv_blocks_per_cu_cap(dev, Ns[i], occ, p.xdirect);
    const int64_t cap = static_cast<int64_t>(dev.num_cu) * per_cu;
    const int g = static_cast<int>(blocks_needed < cap ? blocks_needed : cap);
    if (grids) grids[i] = g;
    p.grid += g;
  }
  return p;
}

QmvPlan qmv_plan(const DeviceInfo& dev, int64_t N, int64_t K, int bits, bool sb_bf16, int act, int mt) {
  return qmv_plan_group(dev, &N, &K, 1, bits, sb_bf16, act, mt, nullptr);
}

hipError_t launch_qmv_group(const QmvProblem* probs, int count, int bits, int glog2, bool sb_bf16,
                            int act, const DeviceInfo& dev, int mt, hipStream_t stream) {
  int64_t Ns[kMaxGroup], Ks[kMaxGroup];
  int grids[kMaxGroup];
  for (int i = 0; i < count; ++i) {
    Ns[i] = probs[i].N;
    Ks[i] = probs[i].K;
  }
  const QmvPlan p = qmv_plan_group(dev, Ns, Ks, count, bits, sb_bf16, act, mt, grids);
  if (p.lds > 65536) {
    hipError_t e = ensure_dynamic_lds(p.kernel, p.lds);
    if (e != hipSuccess) return e;
  }
  QmvBatch batch{};
  batch.glog2 = glog2;
  int begin = 0;
  for (int i = 0; i < kMaxGroup; ++i) batch.block_end[i] = INT_MAX;
  for (int i = 0; i < count; ++i) {
    QmvSlot& q = i == 0 ? batch.first : batch.rest[i - 1];
    q.x = probs[i].x;
    q.w = probs[i].w;
    q.s = probs[i].s;
    q.b = probs[i].b;
    q.y = probs[i].y;
    q.ob = probs[i].ob;
    q.N = static_cast<int>(probs[i].N);
    q.K = static_cast<int>(probs[i].K);
    q.block_begin = begin;
    q.nblk = grids[i];
    begin += grids[i];
    batch.block_end[i] = begin;
  }
  void* args[] = {&batch};
  return hipLaunchKernel(p.kernel, dim3(begin), dim3(kQmvBlock), args, p.lds, stream);
}

hipError_t launch_qmv_slice(const QmvArgs& a, const DeviceInfo& dev, int mt) {
  QmvProblem pr{a.x, a.w, a.s, a.b, a.y, a.ob, a.N, a.K};
  return launch_qmv_group(&pr, 1, a.bits, a.glog2, a.sb_bf16, a.act, dev, mt, a.stream);
}

}  // namespace mxq
