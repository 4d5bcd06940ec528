// extern "C" entry points of libmxq: argument validation (fail-fast, before
// any launch -- the spirit of mlxcel #574's "fail fast instead of faulting
// mid-run" guards in "What is already in-tree"), dispatch, and the host packer.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/mxq.h"
#include "mxq_internal.h"

namespace {

thread_local std::string g_last_error;

mxq_status fail(mxq_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : -1; }

// activation modes of the decode kernel (mxq::QmvArgs::act)
constexpr int kActF16 = 0, kActBF16 = 1, kActI8 = 2;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
mxq::DeviceInfo g_dev[kMaxDevices];
// kernels whose dynamic-LDS limit was raised, and cached occupancies, per device
std::set<std::tuple<const void*, int, size_t>>* g_lds_done = nullptr;
std::map<std::tuple<const void*, int, int, size_t>, int>* g_occ = nullptr;

// Shared validation of the fused entry points; fills the common fields.
mxq_status check_fused(const char* who, const void* x, const uint32_t* w, const void* scales,
                       const void* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                       int group_size, mxq_dtype sb_dtype) {
  const std::string f(who);
  if (M < 0 || N < 0 || K < 0) return fail(MXQ_ERR_INVALID_ARG, f + ": M, N and K must be >= 0");
  if (bits != 4 && bits != 8) return fail(MXQ_ERR_UNSUPPORTED, f + ": bits must be 4 or 8");
  if (log2_group(group_size) < 0)
    return fail(MXQ_ERR_UNSUPPORTED, f + ": group_size must be 32, 64 or 128");
  if (K % group_size != 0) return fail(MXQ_ERR_UNSUPPORTED, f + ": K must be a multiple of group_size");
  if (sb_dtype != MXQ_F16 && sb_dtype != MXQ_BF16)
    return fail(MXQ_ERR_UNSUPPORTED, f + ": scales/biases must be MXQ_F16 or MXQ_BF16");
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(MXQ_ERR_UNSUPPORTED, f + ": M, N and K must each fit in 32 bits");
  if (M == 0 || N == 0) return MXQ_OK;
  if (!y) return fail(MXQ_ERR_INVALID_ARG, f + ": y must not be null");
  if (K > 0 && (!x || !w || !scales || !biases))
    return fail(MXQ_ERR_INVALID_ARG, f + ": x, w, scales and biases must not be null");
  if (K > 0 && !aligned(w, 16)) return fail(MXQ_ERR_MISALIGNED, f + ": w must be 16-byte aligned");
  if (!aligned(x, 2) || !aligned(y, 2) || (K > 0 && (!aligned(scales, 2) || !aligned(biases, 2))))
    return fail(MXQ_ERR_MISALIGNED, f + ": x, y, scales and biases must be 2-byte aligned");
  return MXQ_OK;
}

mxq_status hip_fail(const char* who, hipError_t e) {
  return fail(MXQ_ERR_HIP, std::string(who) + ": " + hipGetErrorName(e) + ": " + hipGetErrorString(e));
}

// Row counts the K-split few-row kernel takes (its shape test aside).
// Two rows: the K-split kernel up to K = 3072 (N = 65536: 24.5 against 32.7
// us); at K = 4096 the two kernels trade places with N, and in K chunks the
// decode kernel ties or wins.
bool qsmk_rows(int64_t M, int64_t K) { return M >= 3 || (M == 2 && K <= 3072); }

// Whether the K-split kernel may run K in chunks on this stream: they need the
// cached split workspace, which a stream being captured into a graph must not
// use (such calls keep the other kernels).  Only asked when K needs chunks.
bool qsmk_chunks_ok(int64_t K, void* stream) {
  if (K <= 4096) return true;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cap == hipStreamCaptureStatusNone;
}

// A caller-provided split workspace (the fixed scratch of mxq_qmm_noalloc):
// calls given one never allocate, may run K in chunks under graph capture,
// and are rejected when they would need more than it holds.
struct FixedWs {
  float* ptr;
  size_t bytes;
};

mxq_status scratch_too_small(const char* who, size_t need, size_t have) {
  return fail(MXQ_ERR_UNSUPPORTED, std::string(who) + ": this call needs " + std::to_string(need) +
                                       " bytes of scratch for its partial results; the fixed scratch holds " +
                                       std::to_string(have));
}

// M-sliced qmv over the whole M range.
mxq_status run_qmv(const char* who, const void* x, const uint32_t* w, const void* scales,
                   const void* biases, const void* out_bias, void* y, int64_t M, int64_t N, int64_t K,
                   int bits, int group_size, mxq_dtype sb_dtype, int act, void* stream,
                   const FixedWs* fws = nullptr) {
  mxq::DeviceInfo dev;
  hipError_t e = mxq::device_info(&dev);
  if (e != hipSuccess) return hip_fail(who, e);
  int mt_max = 8;
  while (mt_max > 1 && mxq::qmv_lds_need(bits, mt_max, K) > dev.lds_per_block) mt_max--;
  if (mxq::qmv_lds_need(bits, 1, K) > dev.lds_per_block)
    return fail(MXQ_ERR_UNSUPPORTED, std::string(who) + ": K too large for the activation staging buffer");
  mxq::QmvArgs a{};
  a.w = w;
  a.s = static_cast<const uint16_t*>(scales);
  a.b = static_cast<const uint16_t*>(biases);
  a.ob = static_cast<const uint16_t*>(out_bias);
  a.N = N;
  a.K = K;
  a.bits = bits;
  a.glog2 = log2_group(group_size);
  a.sb_bf16 = sb_dtype == MXQ_BF16;
  a.act = act;
  a.rows_per_wave = 0;
  a.stream = static_cast<hipStream_t>(stream);
  // A few rows of f16 activations go to the matrix cores when the shape fills
  // the GPU (qsmk_shape): the K-split kernel for 4- or 8-bit codes, group 64
  // or 128, K from 512 (in chunks beyond 4096; K not a multiple of 512, or
  // scales / biases not 16-byte aligned, on its ragged variant), from 3 rows,
  // or from 2 when K <= 3072 (qsmk_rows: there the decode kernel's two-row
  // variant is slower; measured); else the 16-row-block kernel for 9..16 rows
  // (one launch instead of two 8-row decode launches).  Both read x with
  // 16-byte loads.
  // int8 activations take the K-split kernel's integer-MFMA variant from 3
  // rows, unchunked (K <= 4096: one row scale covers all of K); the decode
  // kernel's v_dot4 path is VALU-bound beyond a row or two.  At two rows the
  // two kernels trade places with N (K = 2048: N = 8192 7.6 against 8.8 us on
  // the K-split kernel, which quantizes x in every workgroup; lm_head 26.4
  // against 26.1 us), so two rows stay on the decode kernel.  If the K-chunk
  // workspace cannot be had, the call falls through to the kernels below.
  const bool few_i8 = act == kActI8 && M >= 3;
  if ((act == kActF16 ? qsmk_rows(M, K) : few_i8) && aligned(x, 16) &&
      mxq::qsmk_shape(M, N, K, bits, group_size, act == kActF16 && (fws || qsmk_chunks_ok(K, stream)), dev)) {
    a.x = static_cast<const uint16_t*>(x);
    a.y = static_cast<uint16_t*>(y);
    a.x_vec = 1;
    if (fws) {
      int nw = 0, chunks = 0;
      mxq::qsmk_split(K, &nw, &chunks);
      const size_t need = chunks > 1 ? static_cast<size_t>(chunks) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4 : 0;
      if (need > fws->bytes) return scratch_too_small(who, need, fws->bytes);
      a.fixed_ws = fws->ptr;
      a.fixed_ws_bytes = fws->bytes;
    }
    e = mxq::launch_qsmk(a, static_cast<int>(M), dev);
    if (e != hipErrorOutOfMemory) return e == hipSuccess ? MXQ_OK : hip_fail(who, e);
    (void)hipGetLastError();  // no workspace for the K chunks: nothing was enqueued
  }
  if (act == kActF16 && aligned(x, 16) && mxq::qsm_shape(M, N, K, bits, group_size, dev)) {
    a.x = static_cast<const uint16_t*>(x);
    a.y = static_cast<uint16_t*>(y);
    a.x_vec = 1;
    e = mxq::launch_qsm(a, static_cast<int>(M), dev);
    return e == hipSuccess ? MXQ_OK : hip_fail(who, e);
  }
  for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
    const int mt = static_cast<int>((M - m0) < mt_max ? (M - m0) : mt_max);
    a.x = static_cast<const uint16_t*>(x) + m0 * K;
    a.y = static_cast<uint16_t*>(y) + m0 * N;
    a.x_vec = aligned(a.x, 16) ? 1 : 0;
    e = mxq::launch_qmv_slice(a, dev, mt);
    if (e != hipSuccess) return hip_fail(who, e);
  }
  return MXQ_OK;
}

// Grouped qmv over problems that all passed validation and have N, K > 0.
mxq_status run_qmv_grouped(const char* who, const mxq_qmv_problem* pr, int count, int64_t M, int bits,
                           int group_size, mxq_dtype sb_dtype, void* stream) {
  mxq::DeviceInfo dev;
  hipError_t e = mxq::device_info(&dev);
  if (e != hipSuccess) return hip_fail(who, e);
  int64_t kmax = 0;
  for (int i = 0; i < count; ++i) kmax = pr[i].K > kmax ? pr[i].K : kmax;
  if (mxq::qmv_lds_need(bits, 1, kmax) > dev.lds_per_block)
    return fail(MXQ_ERR_UNSUPPORTED, std::string(who) + ": K too large for the activation staging buffer");
  int mt_max = 8;
  while (mt_max > 1 && mxq::qmv_lds_need(bits, mt_max, kmax) > dev.lds_per_block) mt_max--;
  mxq::QmvProblem chunk[mxq::kMaxGroup];
  for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
    const int mt = static_cast<int>((M - m0) < mt_max ? (M - m0) : mt_max);
    for (int c0 = 0; c0 < count; c0 += mxq::kMaxGroup) {
      const int n = (count - c0) < mxq::kMaxGroup ? (count - c0) : mxq::kMaxGroup;
      for (int i = 0; i < n; ++i) {
        const mxq_qmv_problem& q = pr[c0 + i];
        chunk[i] = mxq::QmvProblem{static_cast<const uint16_t*>(q.x) + m0 * q.K, q.w,
                                   static_cast<const uint16_t*>(q.scales),
                                   static_cast<const uint16_t*>(q.biases),
                                   static_cast<uint16_t*>(q.y) + m0 * q.N, nullptr, q.N, q.K};
      }
      e = mxq::launch_qmv_group(chunk, n, bits, log2_group(group_size), sb_dtype == MXQ_BF16, kActF16, dev, mt,
                                static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(who, e);
    }
  }
  return MXQ_OK;
}

// Validated fused call with M, N > 0: qmv kernel for small M (or shapes the
// MFMA kernel does not take), MFMA kernel otherwise; out_bias may be null.
mxq_status run_matmul(const char* who, const void* x, const uint32_t* w, const void* scales,
                      const void* biases, const void* out_bias, void* y, int64_t M, int64_t N, int64_t K,
                      int bits, int group_size, mxq_dtype sb_dtype, int act, void* stream,
                      const FixedWs* fws = nullptr) {
  if (K == 0) {
    hipError_t e = mxq::launch_fill_rows(static_cast<uint16_t*>(y), static_cast<const uint16_t*>(out_bias), M, N,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MXQ_OK : hip_fail(who, e);
  }
  // The MFMA kernel stages x with 16-byte loads and walks K in stages of 64.
  // int8 activations from 17 rows take the integer prefill kernel (below);
  // other int8 calls and the few-row shapes of f16 activations (qsmk_rows and
  // qsmk_shape) take run_qmv's routing: the K-split matrix-core kernel where
  // it applies, else the decode kernel in 8-row slices.
  mxq::DeviceInfo dev;
  hipError_t e = mxq::device_info(&dev);
  if (e != hipSuccess) return hip_fail(who, e);
  const bool few = act == kActF16 && qsmk_rows(M, K) &&
                   mxq::qsmk_shape(M, N, K, bits, group_size, fws || qsmk_chunks_ok(K, stream), dev);
  // int8 activations from 17 rows: the integer-MFMA prefill kernel (x
  // quantized once into a workspace, W read once); without a workspace, and
  // for fewer rows, run_qmv's routing.
  if (act == kActI8 && !fws && mxq::qmm_a8_shape(M, K) && aligned(x, 16)) {
    mxq::QmmA8Args a8{};
    a8.x = static_cast<const uint16_t*>(x);
    a8.w = w;
    a8.s = static_cast<const uint16_t*>(scales);
    a8.b = static_cast<const uint16_t*>(biases);
    a8.y = static_cast<uint16_t*>(y);
    a8.ob = static_cast<const uint16_t*>(out_bias);
    a8.M = M;
    a8.N = N;
    a8.K = K;
    a8.bits = bits;
    a8.group_size = group_size;
    a8.sb_bf16 = sb_dtype == MXQ_BF16;
    a8.stream = static_cast<hipStream_t>(stream);
    e = mxq::launch_qmm_a8(a8, dev);
    if (e != hipErrorOutOfMemory) return e == hipSuccess ? MXQ_OK : hip_fail(who, e);
    (void)hipGetLastError();  // no workspace: nothing was enqueued
  }
  if (act == kActI8 || few || !mxq::qmm_mfma_shape(M, K) || !aligned(x, 16))
    return run_qmv(who, x, w, scales, biases, out_bias, y, M, N, K, bits, group_size, sb_dtype, act, stream, fws);
  mxq::QmmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = w;
  a.s = static_cast<const uint16_t*>(scales);
  a.b = static_cast<const uint16_t*>(biases);
  a.y = static_cast<uint16_t*>(y);
  a.ob = static_cast<const uint16_t*>(out_bias);
  a.M = M;
  a.N = N;
  a.K = K;
  a.bits = bits;
  a.group_size = group_size;
  a.sb_bf16 = sb_dtype == MXQ_BF16;
  a.x_bf16 = act == kActBF16;
  a.stream = static_cast<hipStream_t>(stream);
  if (fws) {
    const mxq::QmmTile tl = mxq::qmm_pick_tile(M, N, K, dev);
    const bool split = tl.mb == 2 && tl.splits > 1 && (M * N) % 4 == 0;
    const size_t need = split ? static_cast<size_t>(tl.splits) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4 : 0;
    if (need > fws->bytes) return scratch_too_small(who, need, fws->bytes);
    a.fixed_ws = fws->ptr;
    a.fixed_ws_bytes = fws->bytes;
  }
  e = mxq::launch_qmm(a, dev);
  return e == hipSuccess ? MXQ_OK : hip_fail(who, e);
}

}  // namespace

namespace mxq {

hipError_t device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.device != dev) {
    int cu = 0, lds_blk = 0, lds_cu = 0;
    if ((e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&lds_blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) != hipSuccess)
      lds_cu = lds_blk;
    d.num_cu = cu > 0 ? cu : 1;
    d.lds_per_block = static_cast<size_t>(lds_blk > 0 ? lds_blk : 65536);
    d.lds_per_cu = static_cast<size_t>(lds_cu > 0 ? lds_cu : d.lds_per_block);
    d.device = dev;
  }
  *out = d;
  return hipSuccess;
}

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(kernel, dev, bytes);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_lds_done) g_lds_done = new std::set<std::tuple<const void*, int, size_t>>();
    if (g_lds_done->count(key)) return hipSuccess;
  }
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  g_lds_done->insert(key);
  return hipSuccess;
}

int occupancy_blocks(const void* kernel, int threads, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  const auto key = std::make_tuple(kernel, dev, threads, lds);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_occ) g_occ = new std::map<std::tuple<const void*, int, int, size_t>, int>();
    const auto it = g_occ->find(key);
    if (it != g_occ->end()) return it->second;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, lds) != hipSuccess || nb < 1) {
    (void)hipGetLastError();
    nb = 1;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  (*g_occ)[key] = nb;
  return nb;
}

}  // namespace mxq

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_str(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_ERR_INVALID_ARG: return "MXQ_ERR_INVALID_ARG";
    case MXQ_ERR_UNSUPPORTED: return "MXQ_ERR_UNSUPPORTED";
    case MXQ_ERR_MISALIGNED: return "MXQ_ERR_MISALIGNED";
    case MXQ_ERR_HIP: return "MXQ_ERR_HIP";
  }
  return "MXQ_ERR_UNKNOWN";
}

const char* mxq_last_error(void) { return g_last_error.c_str(); }

mxq_status mxq_qmv(const void* x, const uint32_t* w, const void* scales, const void* biases,
                   void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                   mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_qmv", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  if (K == 0) {
    hipError_t e = mxq::launch_zero_fill(static_cast<uint16_t*>(y), M * N, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MXQ_OK : hip_fail("mxq_qmv", e);
  }
  return run_qmv("mxq_qmv", x, w, scales, biases, nullptr, y, M, N, K, bits, group_size, sb_dtype, kActF16, stream);
}

mxq_status mxq_qmv_grouped(const mxq_qmv_problem* problems, int count, int64_t M, int bits,
                           int group_size, mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  if (count < 0) return fail(MXQ_ERR_INVALID_ARG, "mxq_qmv_grouped: count must be >= 0");
  if (count > 0 && !problems) return fail(MXQ_ERR_INVALID_ARG, "mxq_qmv_grouped: problems is null");
  std::vector<mxq_qmv_problem> live;
  for (int i = 0; i < count; ++i) {
    const mxq_qmv_problem& q = problems[i];
    const std::string who = "mxq_qmv_grouped[" + std::to_string(i) + "]";
    mxq_status st = check_fused(who.c_str(), q.x, q.w, q.scales, q.biases, q.y, M, q.N, q.K, bits,
                                group_size, sb_dtype);
    if (st != MXQ_OK) return st;
    if (M > 0 && q.N > 0) live.push_back(q);
  }
  std::vector<mxq_qmv_problem> work;
  for (const mxq_qmv_problem& q : live) {
    if (q.K == 0) {
      hipError_t e = mxq::launch_zero_fill(static_cast<uint16_t*>(q.y), M * q.N, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail("mxq_qmv_grouped", e);
    } else {
      work.push_back(q);
    }
  }
  if (work.empty()) return MXQ_OK;
  return run_qmv_grouped("mxq_qmv_grouped", work.data(), static_cast<int>(work.size()), M, bits,
                         group_size, sb_dtype, stream);
}

mxq_status mxq_qmm(const void* x, const uint32_t* w, const void* scales, const void* biases,
                   void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                   mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_qmm", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  return run_matmul("mxq_qmm", x, w, scales, biases, nullptr, y, M, N, K, bits, group_size, sb_dtype, kActF16,
                    stream);
}

mxq_status mxq_qmm_noalloc(const void* x, const uint32_t* w, const void* scales, const void* biases,
                           void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                           mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_qmm_noalloc", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  FixedWs fws{nullptr, mxq::kStaticScratchBytes};
  const hipError_t e = mxq::static_scratch(&fws.ptr);
  if (e != hipSuccess) return hip_fail("mxq_qmm_noalloc", e);
  return run_matmul("mxq_qmm_noalloc", x, w, scales, biases, nullptr, y, M, N, K, bits, group_size, sb_dtype,
                    kActF16, stream, &fws);
}

mxq_status mxq_linear(const void* x, const uint32_t* w, const void* scales, const void* biases,
                      const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      int group_size, mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_linear", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  if (out_bias && !aligned(out_bias, 2))
    return fail(MXQ_ERR_MISALIGNED, "mxq_linear: out_bias must be 2-byte aligned");
  return run_matmul("mxq_linear", x, w, scales, biases, out_bias, y, M, N, K, bits, group_size, sb_dtype,
                    kActF16, stream);
}

mxq_status mxq_linear_act(const void* x, const uint32_t* w, const void* scales, const void* biases,
                          const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                          int group_size, mxq_dtype sb_dtype, mxq_dtype act_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_linear_act", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK) return st;
  if (act_dtype != MXQ_F16 && act_dtype != MXQ_BF16)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_linear_act: act_dtype must be MXQ_F16 or MXQ_BF16");
  if (M == 0 || N == 0) return MXQ_OK;
  if (out_bias && !aligned(out_bias, 2))
    return fail(MXQ_ERR_MISALIGNED, "mxq_linear_act: out_bias must be 2-byte aligned");
  return run_matmul("mxq_linear_act", x, w, scales, biases, out_bias, y, M, N, K, bits, group_size, sb_dtype,
                    act_dtype == MXQ_BF16 ? kActBF16 : kActF16, stream);
}

mxq_status mxq_linear_a8(const void* x, const uint32_t* w, const void* scales, const void* biases,
                         const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                         int group_size, mxq_dtype sb_dtype, void* stream) {
  g_last_error.clear();
  mxq_status st = check_fused("mxq_linear_a8", x, w, scales, biases, y, M, N, K, bits, group_size, sb_dtype);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  if (out_bias && !aligned(out_bias, 2))
    return fail(MXQ_ERR_MISALIGNED, "mxq_linear_a8: out_bias must be 2-byte aligned");
  return run_matmul("mxq_linear_a8", x, w, scales, biases, out_bias, y, M, N, K, bits, group_size, sb_dtype,
                    kActI8, stream);
}

mxq_status mxq_dequant(const uint32_t* w, const void* scales, const void* biases, void* out,
                       int64_t N, int64_t K, int bits, int group_size, mxq_dtype sb_dtype,
                       mxq_dtype out_dtype, void* stream) {
  g_last_error.clear();
  if (N < 0 || K < 0) return fail(MXQ_ERR_INVALID_ARG, "mxq_dequant: N and K must be >= 0");
  if (bits != 4 && bits != 8) return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: bits must be 4 or 8");
  if (log2_group(group_size) < 0)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: group_size must be 32, 64 or 128");
  if (K % group_size != 0) return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: K must be a multiple of group_size");
  if (sb_dtype != MXQ_F16 && sb_dtype != MXQ_BF16)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: scales/biases must be MXQ_F16 or MXQ_BF16");
  if (out_dtype != MXQ_F16 && out_dtype != MXQ_BF16 && out_dtype != MXQ_F32)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: out_dtype must be MXQ_F16, MXQ_BF16 or MXQ_F32");
  if (N > INT32_MAX || K > INT32_MAX) return fail(MXQ_ERR_UNSUPPORTED, "mxq_dequant: N and K must fit in 32 bits");
  if (N == 0 || K == 0) return MXQ_OK;
  if (!w || !scales || !biases || !out) return fail(MXQ_ERR_INVALID_ARG, "mxq_dequant: null pointer");
  if (!aligned(w, 16) || !aligned(out, 16))
    return fail(MXQ_ERR_MISALIGNED, "mxq_dequant: w and out must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(biases, 2))
    return fail(MXQ_ERR_MISALIGNED, "mxq_dequant: scales and biases must be 2-byte aligned");
  mxq::DeviceInfo dev;
  hipError_t e = mxq::device_info(&dev);
  if (e != hipSuccess) return hip_fail("mxq_dequant", e);
  mxq::DequantArgs a{};
  a.w = w;
  a.s = static_cast<const uint16_t*>(scales);
  a.b = static_cast<const uint16_t*>(biases);
  a.out = out;
  a.N = N;
  a.K = K;
  a.bits = bits;
  a.glog2 = log2_group(group_size);
  a.sb_bf16 = sb_dtype == MXQ_BF16;
  a.out_dtype = static_cast<int>(out_dtype);
  a.stream = static_cast<hipStream_t>(stream);
  e = mxq::launch_dequant(a, dev);
  return e == hipSuccess ? MXQ_OK : hip_fail("mxq_dequant", e);
}

const char* mxq_describe(const char* op, int64_t M, int64_t N, int64_t K, int bits,
                         int group_size, mxq_dtype sb_dtype) {
  thread_local std::string desc;
  const std::string o = op ? op : "";
  if ((o != "qmv" && o != "qmm" && o != "a8") || M <= 0 || N <= 0 || K <= 0 || (bits != 4 && bits != 8) ||
      log2_group(group_size) < 0 || K % group_size != 0 || (sb_dtype != MXQ_F16 && sb_dtype != MXQ_BF16)) {
    desc = "invalid";
    return desc.c_str();
  }
  mxq::DeviceInfo dev;
  if (mxq::device_info(&dev) != hipSuccess) {
    desc = "no device";
    return desc.c_str();
  }
  const char* sb = sb_dtype == MXQ_BF16 ? "bf16" : "f16";
  const bool a8 = o == "a8";
  if ((a8 ? M >= 3 : qsmk_rows(M, K)) && mxq::qsmk_shape(M, N, K, bits, group_size, !a8, dev)) {
    int nw = 0, chunks = 0;
    mxq::qsmk_split(K, &nw, &chunks);
    desc = "qsmk_kernel<bits=" + std::to_string(bits) + ",sb=" + std::string(sb) + ",gs=" +
           std::to_string(group_size) + ",m=" + std::to_string(M) + ",waves=" + std::to_string(nw) +
           (a8 ? ",act=i8" : "") + (chunks > 1 ? ",kchunks=" + std::to_string(chunks) : std::string()) +
           (K % 512 != 0 ? ",ragged" : "") + (mxq::qsmk_xstage(M, a8) ? ",xstage" : "") +
           "> block=" + std::to_string(64 * nw) + " lds=" + std::to_string(mxq::qsmk_lds_bytes(nw, bits, mxq::qsmk_xstage(M, a8))) +
           (chunks > 1 ? "; qmm_split_reduce_kernel" : "");
    return desc.c_str();
  }
  if (a8 && mxq::qmm_a8_shape(M, K)) {
    const mxq::QmmA8Plan p = mxq::qmm_a8_plan(M, N, K, group_size, dev);
    desc = "quant_rows_i8_kernel grid=" + std::to_string(M) + " block=256; qmm_a8_kernel<bits=" + std::to_string(bits) +
           ",sb=" + sb + ",gs=" + std::to_string(group_size) + ",tile=128x128" +
           (p.splits > 1 ? ",ksplit=" + std::to_string(p.splits) : std::string()) + "> grid=" +
           std::to_string(static_cast<int64_t>(p.tiles_m) * p.tiles_n * p.splits) +
           " block=512 lds=" + std::to_string(mxq::qmm_a8_lds_bytes()) +
           (p.splits > 1 ? "; qmm_split_reduce_kernel" : "");
    return desc.c_str();
  }
  const bool mfma = o == "qmm" && mxq::qmm_mfma_shape(M, K);
  if (mfma) {
    const mxq::QmmTile tl = mxq::qmm_pick_tile(M, N, K, dev);
    const int64_t bm = 64 * tl.mb, bn = 64 * tl.nb;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    desc = "qmm_kernel<bits=" + std::to_string(bits) + ",sb=" + sb + ",gs=" + std::to_string(group_size) +
           ",tile=" + std::to_string(bm) + "x" + std::to_string(bn) +
           (tl.splits > 1 ? ",ksplit=" + std::to_string(tl.splits) : std::string()) +
           "> grid=" + std::to_string(tiles * tl.splits) + " block=512";
    return desc.c_str();
  }
  if (!a8 && mxq::qsm_shape(M, N, K, bits, group_size, dev)) {
    desc = "qsm_kernel<bits=" + std::to_string(bits) + ",sb=" + sb + ",m=" + std::to_string(M) + "> grid=" +
           std::to_string((N + 255) / 256) + " block=256 lds=" +
           std::to_string(mxq::qsm_lds_bytes(static_cast<int>(M), static_cast<int>(K)));
    return desc.c_str();
  }
  int mt_max = 8;
  while (mt_max > 1 && mxq::qmv_lds_need(bits, mt_max, K) > dev.lds_per_block) mt_max--;
  desc.clear();
  for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
    const int mt = static_cast<int>((M - m0) < mt_max ? (M - m0) : mt_max);
    const mxq::QmvPlan p = mxq::qmv_plan(dev, N, K, bits, sb_dtype == MXQ_BF16, a8 ? kActI8 : kActF16, mt);
    if (!desc.empty()) desc += "; ";
    desc += "qmv_kernel<bits=" + std::to_string(bits) + ",sb=" + sb + ",mt=" + std::to_string(mt) +
            ",rows=" + std::to_string(p.rows) + (p.xdirect ? ",xreg" : "") + (a8 ? ",act=i8" : "") +
            "> grid=" + std::to_string(p.grid) +
            " block=256 lds=" + std::to_string(p.lds);
  }
  return desc.c_str();
}

mxq_status mxq_read_probe(const void* buf, int64_t bytes, void* out, void* stream) {
  g_last_error.clear();
  if (bytes < 0 || bytes % 16 != 0)
    return fail(MXQ_ERR_INVALID_ARG, "mxq_read_probe: bytes must be a non-negative multiple of 16");
  if (bytes == 0) return MXQ_OK;
  if (!buf || !out) return fail(MXQ_ERR_INVALID_ARG, "mxq_read_probe: null pointer");
  if (!aligned(buf, 16) || !aligned(out, 4))
    return fail(MXQ_ERR_MISALIGNED, "mxq_read_probe: buf must be 16-byte and out 4-byte aligned");
  mxq::DeviceInfo dev;
  hipError_t e = mxq::device_info(&dev);
  if (e != hipSuccess) return hip_fail("mxq_read_probe", e);
  e = mxq::launch_read_probe(buf, bytes, static_cast<uint32_t*>(out), static_cast<hipStream_t>(stream), dev);
  return e == hipSuccess ? MXQ_OK : hip_fail("mxq_read_probe", e);
}

mxq_status mxq_release_workspaces(void) {
  g_last_error.clear();
  (void)mxq::split_workspace_release_all();
  return MXQ_OK;
}

int64_t mxq_workspace_bytes(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return static_cast<int64_t>(mxq::split_workspace_cached_bytes(dev));
}

const char* mxq_describe_grouped(const mxq_qmv_problem* problems, int count, int64_t M, int bits,
                                 int group_size, mxq_dtype sb_dtype) {
  thread_local std::string desc;
  if (count <= 0 || !problems || M <= 0 || (bits != 4 && bits != 8) || log2_group(group_size) < 0 ||
      (sb_dtype != MXQ_F16 && sb_dtype != MXQ_BF16)) {
    desc = "invalid";
    return desc.c_str();
  }
  // the problems mxq_qmv_grouped launches: N > 0 and K > 0 (K = 0 is a fill)
  std::vector<int64_t> Ns, Ks;
  for (int i = 0; i < count; ++i) {
    const mxq_qmv_problem& q = problems[i];
    if (q.N < 0 || q.K < 0 || q.K % group_size != 0) {
      desc = "invalid";
      return desc.c_str();
    }
    if (q.N > 0 && q.K > 0) {
      Ns.push_back(q.N);
      Ks.push_back(q.K);
    }
  }
  if (Ns.empty()) {
    desc = "none";
    return desc.c_str();
  }
  mxq::DeviceInfo dev;
  if (mxq::device_info(&dev) != hipSuccess) {
    desc = "no device";
    return desc.c_str();
  }
  int64_t kmax = 0;
  for (int64_t k : Ks) kmax = k > kmax ? k : kmax;
  int mt_max = 8;
  while (mt_max > 1 && mxq::qmv_lds_need(bits, mt_max, kmax) > dev.lds_per_block) mt_max--;
  const char* sb = sb_dtype == MXQ_BF16 ? "bf16" : "f16";
  desc.clear();
  const int n = static_cast<int>(Ns.size());
  for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
    const int mt = static_cast<int>((M - m0) < mt_max ? (M - m0) : mt_max);
    for (int c0 = 0; c0 < n; c0 += mxq::kMaxGroup) {
      const int cnt = (n - c0) < mxq::kMaxGroup ? (n - c0) : mxq::kMaxGroup;
      const mxq::QmvPlan p = mxq::qmv_plan_group(dev, Ns.data() + c0, Ks.data() + c0, cnt, bits,
                                                 sb_dtype == MXQ_BF16, kActF16, mt, nullptr);
      if (!desc.empty()) desc += "; ";
      desc += "qmv_kernel<bits=" + std::to_string(bits) + ",sb=" + sb + ",mt=" + std::to_string(mt) +
              ",rows=" + std::to_string(p.rows) + (p.xdirect ? ",xreg" : "") + "> problems=" +
              std::to_string(cnt) + " grid=" + std::to_string(p.grid) + " block=256 lds=" + std::to_string(p.lds);
    }
  }
  return desc.c_str();
}

mxq_status mxq_pack(const uint8_t* codes, uint32_t* w, int64_t N, int64_t K, int bits) {
  g_last_error.clear();
  if (bits != 4 && bits != 8) return fail(MXQ_ERR_UNSUPPORTED, "mxq_pack: bits must be 4 or 8");
  if (N < 0 || K < 0) return fail(MXQ_ERR_INVALID_ARG, "mxq_pack: N and K must be >= 0");
  const int per = 32 / bits;
  if (K % per != 0) return fail(MXQ_ERR_UNSUPPORTED, "mxq_pack: K must be a multiple of 32/bits");
  if (N == 0 || K == 0) return MXQ_OK;
  if (!codes || !w) return fail(MXQ_ERR_INVALID_ARG, "mxq_pack: null pointer");
  const uint32_t limit = 1u << bits;
  const int64_t kw = K / per;
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* c = codes + n * K;
    uint32_t* o = w + n * kw;
    for (int64_t j = 0; j < kw; ++j) {
      uint32_t word = 0;
      for (int i = 0; i < per; ++i) {
        const uint32_t v = c[j * per + i];
        if (v >= limit) return fail(MXQ_ERR_INVALID_ARG, "mxq_pack: code does not fit in `bits` bits");
        word |= v << (bits * i);  // field i holds code i: least significant first
      }
      o[j] = word;
    }
  }
  return MXQ_OK;
}

}  // extern "C"
