// Driver for the sanitizer build of libmxq's C-ABI layer (api.cpp and
// workspace.cpp under AddressSanitizer + UndefinedBehaviorSanitizer, with
// the HIP runtime and the kernel launchers replaced by host stand-ins).
//
// It calls every entry point with exact-size host buffers over a spread of
// shapes (the stand-in launchers touch every range a kernel would read or
// write), walks the argument checks with one bad argument at a time, packs
// and unpacks codes, and drives the split workspace cache from several
// streams, devices and threads, including allocation failures.  Exits 0 and
// prints "sanitize driver: ok" when every check holds; a sanitizer report
// ends the process with an error first.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "mxq.h"
#include "mxq_internal.h"

extern "C" void stub_fail_malloc(int on);
extern "C" long stub_live_allocations(void);

#define CHECK(c)                                                                                 \
  do {                                                                                           \
    if (!(c)) {                                                                                  \
      std::fprintf(stderr, "CHECK failed at %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #c, \
                   mxq_last_error());                                                            \
      std::exit(1);                                                                              \
    }                                                                                            \
  } while (0)

namespace {

// an exact-size, 256-byte aligned host allocation (the sanitizer knows its end)
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t n) {
    if (posix_memalign(&p, 256, n ? n : 1) != 0) std::abort();
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  template <typename T>
  T* as(size_t byte_offset = 0) const {
    return reinterpret_cast<T*>(static_cast<char*>(p) + byte_offset);
  }
};

struct Shape {
  int64_t M, N, K;
  int bits, gs;
  mxq_dtype sb;
};

struct Problem {
  Shape s;
  Buf x, w, sc, bi, y, ob, out;
  explicit Problem(const Shape& sh)
      : s(sh),
        x(static_cast<size_t>(sh.M * sh.K * 2) + 16),  // + 16: room for the offset-x case
        w(static_cast<size_t>(sh.N * sh.K * sh.bits / 8)),
        sc(static_cast<size_t>(sh.N * (sh.K / sh.gs) * 2)),
        bi(static_cast<size_t>(sh.N * (sh.K / sh.gs) * 2)),
        y(static_cast<size_t>(sh.M * sh.N * 2)),
        ob(static_cast<size_t>(sh.N * 2)),
        out(static_cast<size_t>(sh.N * sh.K * 4)) {}
};

void* stream_of(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x1000 + 0x40 * i)); }

void run_all_entry_points(const Problem& p, void* st) {
  const Shape& s = p.s;
  const void* x = p.x.p;
  const uint32_t* w = p.w.as<uint32_t>();
  CHECK(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  CHECK(mxq_qmm(x, w, p.sc.p, p.bi.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  CHECK(mxq_linear(x, w, p.sc.p, p.bi.p, nullptr, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  CHECK(mxq_linear(x, w, p.sc.p, p.bi.p, p.ob.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  CHECK(mxq_linear_act(x, w, p.sc.p, p.bi.p, p.ob.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, MXQ_BF16, st) ==
        MXQ_OK);
  CHECK(mxq_linear_a8(x, w, p.sc.p, p.bi.p, p.ob.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  const mxq_status na = mxq_qmm_noalloc(x, w, p.sc.p, p.bi.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st);
  CHECK(na == MXQ_OK || na == MXQ_ERR_UNSUPPORTED);
  // x 2-byte aligned but not 16: the same calls take the narrow-load routes
  const void* x2 = p.x.as<char>(2);
  CHECK(mxq_qmv(x2, w, p.sc.p, p.bi.p, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  CHECK(mxq_linear_a8(x2, w, p.sc.p, p.bi.p, nullptr, p.y.p, s.M, s.N, s.K, s.bits, s.gs, s.sb, st) == MXQ_OK);
  for (mxq_dtype od : {MXQ_F32, MXQ_F16, MXQ_BF16})
    CHECK(mxq_dequant(w, p.sc.p, p.bi.p, p.out.p, s.N, s.K, s.bits, s.gs, s.sb, od, st) == MXQ_OK);
  for (const char* op : {"qmv", "qmm", "a8"}) CHECK(mxq_describe(op, s.M, s.N, s.K, s.bits, s.gs, s.sb) != nullptr);
}

void shapes_sweep() {
  std::mt19937 rng(7);
  const int64_t Ms[] = {0, 1, 2, 3, 5, 8, 9, 12, 16, 17, 33, 64, 130, 512};
  const int64_t NKs[][2] = {{1, 64}, {7, 128}, {300, 1152}, {4096, 2048}, {4100, 4096}, {2048, 8192}, {513, 0},
                            {64, 6144}, {4096, 8192}};
  const int bitss[] = {4, 8};
  const int gss[] = {32, 64, 128};
  int done = 0;
  for (int64_t M : Ms)
    for (const auto& nk : NKs) {
      // two random (bits, group, scale dtype) picks per (M, N, K)
      for (int r = 0; r < 2; ++r) {
        const int bits = bitss[rng() % 2], gs = gss[rng() % 3];
        const mxq_dtype sb = (rng() % 2) ? MXQ_BF16 : MXQ_F16;
        if (nk[1] % gs != 0) continue;
        Problem p(Shape{M, nk[0], nk[1], bits, gs, sb});
        run_all_entry_points(p, stream_of(static_cast<int>(rng() % 6)));
        ++done;
      }
    }
  CHECK(done > 100);
}

void grouped_sweep() {
  std::mt19937 rng(11);
  for (int it = 0; it < 40; ++it) {
    const int count = 1 + static_cast<int>(rng() % 20);
    static const int64_t kMs[] = {1, 2, 3, 9};
    const int64_t M = kMs[rng() % 4];
    const int bits = (rng() % 2) ? 4 : 8;
    std::vector<Problem*> ps;
    std::vector<mxq_qmv_problem> pr;
    for (int i = 0; i < count; ++i) {
      const int64_t N = 1 + static_cast<int64_t>(rng() % 3000);
      const int64_t K = 64 * (1 + static_cast<int64_t>(rng() % 40));
      ps.push_back(new Problem(Shape{M, N, K, bits, 64, MXQ_F16}));
      const Problem& p = *ps.back();
      pr.push_back(mxq_qmv_problem{p.x.p, p.w.as<uint32_t>(), p.sc.p, p.bi.p, p.y.p, N, K});
    }
    CHECK(mxq_qmv_grouped(pr.data(), count, M, bits, 64, MXQ_F16, stream_of(it % 5)) == MXQ_OK);
    CHECK(mxq_describe_grouped(pr.data(), count, M, bits, 64, MXQ_F16) != nullptr);
    for (Problem* p : ps) delete p;
  }
}

// one bad argument at a time: an error status, a message, nothing touched
void argument_checks() {
  Problem p(Shape{4, 256, 512, 4, 64, MXQ_F16});
  const void* x = p.x.p;
  const uint32_t* w = p.w.as<uint32_t>();
  void* st = stream_of(0);
  auto bad = [](mxq_status s) {
    CHECK(s != MXQ_OK);
    CHECK(std::strlen(mxq_last_error()) > 0);
  };
  bad(mxq_qmv(nullptr, w, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, nullptr, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, nullptr, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, nullptr, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, nullptr, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, -1, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, -1, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, -64, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 3, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 48, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, 500, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F32, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, int64_t{1} << 31, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, int64_t{1} << 31, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.p, 4, 256, int64_t{1} << 31, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(p.x.as<char>(1), w, p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));   // x odd
  bad(mxq_qmv(x, p.w.as<uint32_t>(4), p.sc.p, p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));  // w not 16
  bad(mxq_qmv(x, w, p.sc.as<char>(1), p.bi.p, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_qmv(x, w, p.sc.p, p.bi.p, p.y.as<char>(1), 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_linear(x, w, p.sc.p, p.bi.p, p.ob.as<char>(1), p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_linear_act(x, w, p.sc.p, p.bi.p, nullptr, p.y.p, 4, 256, 512, 4, 64, MXQ_F16, MXQ_F32, st));
  bad(mxq_linear_a8(x, w, p.sc.p, p.bi.p, p.ob.as<char>(1), p.y.p, 4, 256, 512, 4, 64, MXQ_F16, st));
  bad(mxq_dequant(w, p.sc.p, p.bi.p, p.out.as<char>(8), 256, 512, 4, 64, MXQ_F16, MXQ_F32, st));
  bad(mxq_dequant(w, p.sc.p, p.bi.p, p.out.p, 256, 512, 4, 64, MXQ_F16, static_cast<mxq_dtype>(7), st));
  bad(mxq_qmv_grouped(nullptr, 1, 1, 4, 64, MXQ_F16, st));
  bad(mxq_qmv_grouped(nullptr, -1, 1, 4, 64, MXQ_F16, st));
  bad(mxq_read_probe(p.x.p, 17, p.y.p, st));
  bad(mxq_read_probe(nullptr, 16, p.y.p, st));
  // K = 0 and M = 0 need no data pointers
  CHECK(mxq_qmv(nullptr, nullptr, nullptr, nullptr, p.y.p, 4, 256, 0, 4, 64, MXQ_F16, st) == MXQ_OK);
  CHECK(mxq_qmv(nullptr, w, p.sc.p, p.bi.p, nullptr, 0, 256, 512, 4, 64, MXQ_F16, st) == MXQ_OK);
  CHECK(mxq_read_probe(p.x.p, 0, p.y.p, st) == MXQ_OK);
  CHECK(mxq_read_probe(p.x.p, 2048, p.y.p, st) == MXQ_OK);
  for (int s = 0; s <= 5; ++s) CHECK(mxq_status_str(static_cast<mxq_status>(s)) != nullptr);
  CHECK(mxq_status_str(static_cast<mxq_status>(99)) != nullptr);
  CHECK(std::strcmp(mxq_describe("nope", 1, 1, 64, 4, 64, MXQ_F16), "invalid") == 0);
  CHECK(mxq_describe(nullptr, 1, 1, 64, 4, 64, MXQ_F16) != nullptr);
  CHECK(mxq_abi_version() == MXQ_ABI_VERSION);
}

void pack_checks() {
  std::mt19937 rng(3);
  for (int bits : {4, 8}) {
    for (int it = 0; it < 60; ++it) {
      const int64_t N = 1 + static_cast<int64_t>(rng() % 40);
      const int64_t K = (32 / bits) * (1 + static_cast<int64_t>(rng() % 40));
      Buf codes(static_cast<size_t>(N * K));
      Buf words(static_cast<size_t>(N * K * bits / 8));
      uint8_t* c = codes.as<uint8_t>();
      for (int64_t i = 0; i < N * K; ++i) c[i] = static_cast<uint8_t>(rng() & ((1u << bits) - 1));
      CHECK(mxq_pack(c, words.as<uint32_t>(), N, K, bits) == MXQ_OK);
      const uint32_t* wv = words.as<uint32_t>();
      const int per = 32 / bits;
      for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
          const uint32_t word = wv[(n * K + k) / per];
          CHECK(((word >> (bits * (k % per))) & ((1u << bits) - 1)) == c[n * K + k]);
        }
      if (bits == 4) {
        c[rng() % (N * K)] = 16;  // does not fit
        CHECK(mxq_pack(c, words.as<uint32_t>(), N, K, bits) != MXQ_OK);
      }
    }
  }
  Buf one(64);
  CHECK(mxq_pack(nullptr, one.as<uint32_t>(), 1, 8, 4) != MXQ_OK);
  CHECK(mxq_pack(one.as<uint8_t>(), nullptr, 1, 8, 4) != MXQ_OK);
  CHECK(mxq_pack(one.as<uint8_t>(), one.as<uint32_t>(), 1, 6, 4) != MXQ_OK);
  CHECK(mxq_pack(one.as<uint8_t>(), one.as<uint32_t>(), 1, 8, 5) != MXQ_OK);
  CHECK(mxq_pack(one.as<uint8_t>(), one.as<uint32_t>(), 0, 8, 4) == MXQ_OK);
}

void workspace_checks() {
  std::mt19937 rng(5);
  for (int dev = 0; dev < 2; ++dev) {
    CHECK(hipSetDevice(dev) == hipSuccess);
    size_t largest = 0;
    for (int it = 0; it < 60; ++it) {
      const size_t bytes = 4096 * (1 + rng() % 2048);
      largest = bytes > largest ? bytes : largest;
      std::lock_guard<std::mutex> lk(mxq::split_workspace_mutex());
      float* ws = mxq::split_workspace_locked(dev, static_cast<hipStream_t>(stream_of(static_cast<int>(rng() % 7))),
                                              bytes);
      CHECK(ws != nullptr);
      std::memset(ws, 0xA5, bytes);  // the whole buffer must be ours
    }
    CHECK(mxq::split_workspace_cached_bytes(dev) <= mxq::kWorkspaceEntries * largest);
  }
  CHECK(hipSetDevice(0) == hipSuccess);
  CHECK(mxq_release_workspaces() == MXQ_OK);
  CHECK(mxq_workspace_bytes() == 0);
  CHECK(stub_live_allocations() == 0);

  // allocation failures: the allocating routes fall back and still succeed
  stub_fail_malloc(1);
  {
    Problem qmm(Shape{512, 2048, 8192, 4, 64, MXQ_F16});  // split K
    CHECK(mxq_qmm(qmm.x.p, qmm.w.as<uint32_t>(), qmm.sc.p, qmm.bi.p, qmm.y.p, 512, 2048, 8192, 4, 64, MXQ_F16,
                  stream_of(1)) == MXQ_OK);
    Problem few(Shape{8, 4096, 8192, 4, 64, MXQ_F16});  // K chunks
    CHECK(mxq_qmv(few.x.p, few.w.as<uint32_t>(), few.sc.p, few.bi.p, few.y.p, 8, 4096, 8192, 4, 64, MXQ_F16,
                  stream_of(2)) == MXQ_OK);
    Problem a8(Shape{64, 300, 1152, 4, 64, MXQ_F16});  // int8 prefill workspace
    CHECK(mxq_linear_a8(a8.x.p, a8.w.as<uint32_t>(), a8.sc.p, a8.bi.p, nullptr, a8.y.p, 64, 300, 1152, 4, 64,
                        MXQ_F16, stream_of(3)) == MXQ_OK);
  }
  stub_fail_malloc(0);
  CHECK(mxq_workspace_bytes() == 0);

  // the no-allocation entry point refuses what its fixed scratch cannot hold
  {
    Problem big(Shape{16, 300000, 8192, 4, 64, MXQ_F16});
    CHECK(mxq_qmm_noalloc(big.x.p, big.w.as<uint32_t>(), big.sc.p, big.bi.p, big.y.p, 16, 300000, 8192, 4, 64,
                          MXQ_F16, stream_of(0)) == MXQ_ERR_UNSUPPORTED);
    CHECK(mxq_workspace_bytes() == 0);
  }

  // several threads calling allocating routes on more streams than the cache keeps
  std::vector<std::thread> th;
  for (int t = 0; t < 4; ++t)
    th.emplace_back([t]() {
      std::mt19937 r(100 + t);
      Problem q(Shape{256, 1024, 8192, 4, 64, MXQ_F16});
      Problem a(Shape{64, 512, 2048, 8, 32, MXQ_BF16});
      for (int it = 0; it < 40; ++it) {
        void* st = stream_of(static_cast<int>(r() % 9));
        CHECK(mxq_qmm(q.x.p, q.w.as<uint32_t>(), q.sc.p, q.bi.p, q.y.p, 256, 1024, 8192, 4, 64, MXQ_F16, st) ==
              MXQ_OK);
        CHECK(mxq_linear_a8(a.x.p, a.w.as<uint32_t>(), a.sc.p, a.bi.p, a.ob.p, a.y.p, 64, 512, 2048, 8, 32,
                            MXQ_BF16, st) == MXQ_OK);
        if (r() % 10 == 0) CHECK(mxq_release_workspaces() == MXQ_OK);
      }
    });
  for (auto& x : th) x.join();
  CHECK(mxq_release_workspaces() == MXQ_OK);
  CHECK(stub_live_allocations() == 0);
}

}  // namespace

int main() {
  argument_checks();
  pack_checks();
  shapes_sweep();
  grouped_sweep();
  workspace_checks();
  CHECK(mxq_release_workspaces() == MXQ_OK);
  std::printf("sanitize driver: ok\n");
  return 0;
}
