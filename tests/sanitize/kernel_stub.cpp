// Host-only stand-ins for libmxq's launch and planning functions (the ones
// that live beside the kernels), for the sanitizer build of the C-ABI layer.
// Each launch touches the first and last byte (and one byte per 4 KiB) of
// every range the real kernel reads or writes, computed from its arguments,
// so AddressSanitizer reports any pointer or size the C-ABI layer gets wrong
// (the driver passes exact-size host buffers).  Workspace users take the
// split workspace cache exactly as the real launchers do.
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mxq_internal.h"

namespace {
void touch(const void* p, size_t bytes) {
  if (bytes == 0) return;
  const volatile unsigned char* c = static_cast<const volatile unsigned char*>(p);
  unsigned char acc = c[0] ^ c[bytes - 1];
  for (size_t i = 4096; i < bytes; i += 4096) acc ^= c[i];
  (void)acc;
}
void touch_w(void* p, size_t bytes) {
  if (bytes == 0) return;
  volatile unsigned char* c = static_cast<volatile unsigned char*>(p);
  c[0] = 0;
  c[bytes - 1] = 0;
  for (size_t i = 4096; i < bytes; i += 4096) c[i] = 0;
}
size_t sz(int64_t a, int64_t b, int64_t e) { return static_cast<size_t>(a) * static_cast<size_t>(b) * static_cast<size_t>(e); }
void touch_weights(const uint32_t* w, const uint16_t* s, const uint16_t* b, int64_t N, int64_t K, int bits, int gs) {
  touch(w, sz(N, K * bits / 8, 1));
  touch(s, sz(N, K / gs, 2));
  touch(b, sz(N, K / gs, 2));
}
// stand-in for a launcher that needs `bytes` of split workspace
hipError_t with_workspace(float* fixed, size_t fixed_bytes, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (fixed != nullptr) {
    if (bytes > fixed_bytes) return hipErrorInvalidValue;
    touch_w(fixed, bytes);
    return hipSuccess;
  }
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(mxq::split_workspace_mutex());
  float* ws = mxq::split_workspace_locked(dev, stream, bytes);
  if (ws == nullptr) return hipErrorOutOfMemory;
  touch_w(ws, bytes);
  return hipSuccess;
}
alignas(256) float g_scratch[mxq::kStaticScratchBytes / sizeof(float)];
}  // namespace

namespace mxq {

size_t qmv_lds_need(int bits, int mt, int64_t K) { return static_cast<size_t>(mt) * static_cast<size_t>(K) * 2 + (bits == 8 ? 512 : 256); }

QmvPlan qmv_plan(const DeviceInfo& dev, int64_t N, int64_t K, int bits, bool, int, int mt) {
  QmvPlan p{};
  p.mt = mt;
  p.rows = N >= 65536 ? 4 : 1;
  p.grid = static_cast<int>((N + 4 * p.rows - 1) / (4 * p.rows));
  if (p.grid > 2 * dev.num_cu) p.grid = 2 * dev.num_cu;
  p.xdirect = mt <= 2 && K <= 2048;
  p.lds = p.xdirect ? 0 : qmv_lds_need(bits, mt, K);
  p.kernel = nullptr;
  return p;
}

QmvPlan qmv_plan_group(const DeviceInfo& dev, const int64_t* Ns, const int64_t* Ks, int count, int bits, bool sb,
                       int act, int mt, int* grids) {
  int64_t nsum = 0, kmax = 0;
  for (int i = 0; i < count; ++i) {
    nsum += Ns[i];
    kmax = Ks[i] > kmax ? Ks[i] : kmax;
    if (grids) grids[i] = static_cast<int>((Ns[i] + 15) / 16);  // null: plan only
  }
  return qmv_plan(dev, nsum, kmax, bits, sb, act, mt);
}

hipError_t launch_qmv_slice(const QmvArgs& a, const DeviceInfo&, int mt) {
  touch(a.x, sz(mt, a.K, 2));
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, 1 << a.glog2);
  if (a.ob) touch(a.ob, sz(a.N, 1, 2));
  touch_w(a.y, sz(mt, a.N, 2));
  return hipSuccess;
}

hipError_t launch_qmv_group(const QmvProblem* probs, int count, int bits, int glog2, bool, int, const DeviceInfo&,
                            int mt, hipStream_t) {
  if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
  for (int i = 0; i < count; ++i) {
    const QmvProblem& p = probs[i];
    touch(p.x, sz(mt, p.K, 2));
    touch_weights(p.w, p.s, p.b, p.N, p.K, bits, 1 << glog2);
    if (p.ob) touch(p.ob, sz(p.N, 1, 2));
    touch_w(p.y, sz(mt, p.N, 2));
  }
  return hipSuccess;
}

bool qsm_shape(int64_t M, int64_t N, int64_t K, int, int group_size, const DeviceInfo& dev) {
  return M >= 9 && M <= 16 && group_size >= 64 && K % 64 == 0 && N >= 256 * static_cast<int64_t>(dev.num_cu) / 64;
}
size_t qsm_lds_bytes(int M, int K) { return static_cast<size_t>(M) * (K + 8) * 2 + static_cast<size_t>(K / 64) * 64; }
hipError_t launch_qsm(const QmvArgs& a, int M, const DeviceInfo&) {
  touch(a.x, sz(M, a.K, 2));
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, 1 << a.glog2);
  if (a.ob) touch(a.ob, sz(a.N, 1, 2));
  touch_w(a.y, sz(M, a.N, 2));
  return hipSuccess;
}

bool qsmk_split(int64_t K, int* waves, int* chunks) {
  if (K < 512 || K % 64 != 0) return false;
  const int64_t slices = (K + 511) / 512;  // the last one may be partial (ragged K)
  *chunks = static_cast<int>((slices + 7) / 8);
  *waves = static_cast<int>((slices + *chunks - 1) / *chunks);
  return true;
}
bool qsmk_ragged(int64_t K, const void* s, const void* b) {
  return K % 512 != 0 || (reinterpret_cast<uintptr_t>(s) & 15) != 0 || (reinterpret_cast<uintptr_t>(b) & 15) != 0;
}
bool qsmk_shape(int64_t M, int64_t N, int64_t K, int, int group_size, bool chunks_ok, const DeviceInfo&) {
  int w = 0, c = 0;
  if (M < 2 || M > 16 || group_size < 64 || K % group_size != 0 || !qsmk_split(K, &w, &c)) return false;
  if (c > 1 && (!chunks_ok || (M * N) % 4 != 0)) return false;
  return N >= 4096;
}
size_t qsmk_lds_bytes(int waves, int bits, bool xstage) {
  return static_cast<size_t>(waves) * 16 * (bits == 8 ? 1040 : 528) + 4096 + (xstage ? 1024 : 0);
}
bool qsmk_xstage(int64_t M, bool int8_act) { return !int8_act && M >= 9; }
hipError_t launch_qsmk(const QmvArgs& a, int M, const DeviceInfo&) {
  int w = 0, c = 0;
  qsmk_split(a.K, &w, &c);
  hipError_t e = with_workspace(a.fixed_ws, a.fixed_ws_bytes, c > 1 ? sz(c, M, a.N) * 4 : 0, a.stream);
  if (e != hipSuccess) return e;
  touch(a.x, sz(M, a.K, 2));
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, 1 << a.glog2);
  if (a.ob) touch(a.ob, sz(a.N, 1, 2));
  touch_w(a.y, sz(M, a.N, 2));
  return hipSuccess;
}

QmmTile qmm_pick_tile(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
  const int64_t big = ((M + 127) / 128) * ((N + 127) / 128);
  if (big >= dev.num_cu) return QmmTile{2, 2, 1};
  const int64_t nkt = K / 64;
  int64_t splits = (dev.num_cu + big - 1) / big;
  if (splits > nkt / 8) splits = nkt / 8;
  if (splits >= 2) {
    const int64_t nks = (nkt + splits - 1) / splits;
    return QmmTile{2, 2, static_cast<int>((nkt + nks - 1) / nks)};
  }
  return QmmTile{1, 1, 1};
}
hipError_t launch_qmm(const QmmArgs& a, const DeviceInfo& dev) {
  const QmmTile t = qmm_pick_tile(a.M, a.N, a.K, dev);
  if (t.splits > 1 && (a.M * a.N) % 4 == 0) {
    const hipError_t e = with_workspace(a.fixed_ws, a.fixed_ws_bytes, sz(t.splits, a.M, a.N) * 4, a.stream);
    if (e != hipSuccess && e != hipErrorOutOfMemory) return e;  // no memory: the unsplit kernel
  }
  touch(a.x, sz(a.M, a.K, 2));
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, a.group_size);
  if (a.ob) touch(a.ob, sz(a.N, 1, 2));
  touch_w(a.y, sz(a.M, a.N, 2));
  return hipSuccess;
}

QmmA8Plan qmm_a8_plan(int64_t M, int64_t N, int64_t K, int group_size, const DeviceInfo& dev) {
  QmmA8Plan p{};
  p.tiles_m = static_cast<int>((M + 127) / 128);
  p.tiles_n = static_cast<int>((N + 127) / 128);
  const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n, nkt = K / 64;
  int64_t splits = 1;
  if (tiles < dev.num_cu && (M * N) % 4 == 0) {
    splits = (dev.num_cu + tiles - 1) / tiles;
    if (splits > nkt / 8) splits = nkt / 8;
    if (splits < 1) splits = 1;
  }
  const int64_t nks = (nkt + splits - 1) / splits;
  p.nks = static_cast<int>(nks);
  p.splits = static_cast<int>((nkt + nks - 1) / nks);
  const int rgc = group_size < 64 ? group_size : 64;
  p.xq_bytes = sz(M, K, 1);
  p.xsum_bytes = sz(M, K / rgc, 4);
  p.sx_bytes = sz(M, 1, 4);
  p.part_bytes = p.splits > 1 ? sz(p.splits, M, N) * 4 : 0;
  p.workspace_bytes = p.part_bytes + p.xq_bytes + p.xsum_bytes + p.sx_bytes;
  return p;
}
size_t qmm_a8_lds_bytes() { return 104960; }
hipError_t launch_qmm_a8(const QmmA8Args& a, const DeviceInfo& dev) {
  const QmmA8Plan p = qmm_a8_plan(a.M, a.N, a.K, a.group_size, dev);
  const hipError_t e = with_workspace(nullptr, 0, p.workspace_bytes, a.stream);
  if (e != hipSuccess) return e;
  touch(a.x, sz(a.M, a.K, 2));
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, a.group_size);
  if (a.ob) touch(a.ob, sz(a.N, 1, 2));
  touch_w(a.y, sz(a.M, a.N, 2));
  return hipSuccess;
}

hipError_t launch_dequant(const DequantArgs& a, const DeviceInfo&) {
  touch_weights(a.w, a.s, a.b, a.N, a.K, a.bits, 1 << a.glog2);
  touch_w(a.out, sz(a.N, a.K, a.out_dtype == 2 ? 4 : 2));
  return hipSuccess;
}

hipError_t launch_fill_rows(uint16_t* y, const uint16_t* ob, int64_t M, int64_t N, hipStream_t) {
  if (ob) touch(ob, sz(N, 1, 2));
  touch_w(y, sz(M, N, 2));
  return hipSuccess;
}
hipError_t launch_zero_fill(uint16_t* y, int64_t count, hipStream_t) {
  touch_w(y, sz(count, 1, 2));
  return hipSuccess;
}
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t, const DeviceInfo&) {
  touch(buf, static_cast<size_t>(bytes));
  touch_w(out, 4);
  return hipSuccess;
}
hipError_t launch_split_reduce_f16(const float* part, const uint16_t* ob, uint16_t* y, int64_t M, int64_t N,
                                   int splits, hipStream_t) {
  touch(part, sz(splits, M, N) * 4);
  if (ob) touch(ob, sz(N, 1, 2));
  touch_w(y, sz(M, N, 2));
  return hipSuccess;
}

hipError_t static_scratch(float** out) {
  *out = g_scratch;
  return hipSuccess;
}

}  // namespace mxq
