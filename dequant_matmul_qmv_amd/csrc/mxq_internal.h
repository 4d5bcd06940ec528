// Host-side internals shared by the launch code of libmxq (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <mutex>
#include <stdint.h>

namespace mxq {

struct DeviceInfo {
  int device = -1;
  int num_cu = 0;
  size_t lds_per_block = 0;  // largest dynamic LDS one workgroup may use
  size_t lds_per_cu = 0;
};

// Cached per device; returns hipSuccess and fills `out` for the current device.
hipError_t device_info(DeviceInfo* out);

// Raise a kernel's dynamic-LDS limit once per (kernel, device).
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

// Workgroups of `threads` threads with `lds` bytes of dynamic LDS that fit on
// one compute unit of the current device (at least 1), queried once per
// (kernel, device, threads, lds) and cached: the query costs host time on
// every launch otherwise.
int occupancy_blocks(const void* kernel, int threads, size_t lds);

// Up to kMaxGroup independent qmv problems sharing one launch (bits, group
// size, scale dtype and the activation row count are common).  Passed by value
// as the kernel argument: no device allocation, safe under graph capture.
constexpr int kMaxGroup = 16;
// One problem of a grouped launch: 64 bytes, so a workgroup fetches all of its
// fields with one scalar load once it knows its problem.
struct QmvSlot {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;
  const uint16_t* ob;  // f16 output bias [N] or null
  int N;
  int K;
  int block_begin;     // first block of the grid that works on this problem
  int nblk;            // blocks working on it
};
static_assert(sizeof(QmvSlot) == 64, "one 64-byte scalar load per problem");
// Problem 0 sits next to the block ranges, so single-problem launches (and
// the blocks of a group's first problem) read everything in one round trip.
struct QmvBatch {
  int block_end[kMaxGroup];  // one past the last block of problem p; INT_MAX past count
  QmvSlot first;             // problem 0
  int glog2;
  int pad[15];
  QmvSlot rest[kMaxGroup - 1];  // problems 1 ..
};

struct QmvProblem {
  const uint16_t* x;   // activation bits (f16 or bf16) [M, K] of this slice
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;         // activation bits [M, N] of this slice
  const uint16_t* ob;  // activation bits [N], added to every row of y, or null
  int64_t N, K;
};

struct QmvArgs {
  const uint16_t* x;   // activation bits (f16 or bf16) [M, K] of this slice
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;         // activation bits [M, N] of this slice
  const uint16_t* ob;  // activation bits [N], added to every row of y, or null
  int64_t N, K;
  int bits;
  int glog2;           // log2(group_size)
  bool sb_bf16;
  int act;             // activations: 0 f16, 1 bf16 (x, y, output bias), 2 f16 quantized to int8 per row
  int x_vec;           // x is 16-byte aligned
  int rows_per_wave;   // 0 = pick automatically
  hipStream_t stream;
  float* fixed_ws;        // caller-provided split workspace (no allocation), or null: the cache
  size_t fixed_ws_bytes;
};

size_t qmv_lds_need(int bits, int mt, int64_t K);

// Launch shape of one qmv slice: template MT (activation rows) and R (rows of
// W per wave per step), grid size and dynamic LDS bytes.
struct QmvPlan {
  int mt, rows, grid;
  bool xdirect;  // activations loaded straight into registers (no LDS staging)
  size_t lds;
  const void* kernel;
};
// act: activation mode, 0 f16, 1 bf16, 2 int8 (f16 x quantized per row inside the kernel)
QmvPlan qmv_plan(const DeviceInfo& dev, int64_t N, int64_t K, int bits, bool sb_bf16, int act, int mt);
QmvPlan qmv_plan_group(const DeviceInfo& dev, const int64_t* Ns, const int64_t* Ks, int count, int bits,
                       bool sb_bf16, int act, int mt, int* grids);
hipError_t launch_qmv_slice(const QmvArgs& a, const DeviceInfo& dev, int mt);
// One launch for `count` (<= kMaxGroup) problems with a common mt (rows of x).
hipError_t launch_qmv_group(const QmvProblem* probs, int count, int bits, int glog2, bool sb_bf16,
                            int act, const DeviceInfo& dev, int mt, hipStream_t stream);

// Few-row kernel on the matrix cores (9 <= M <= 16 activation rows, f16
// activations, group size 64 or 128, N large enough to occupy the GPU).
bool qsm_shape(int64_t M, int64_t N, int64_t K, int bits, int group_size, const DeviceInfo& dev);
size_t qsm_lds_bytes(int M, int K);
// All M rows in one launch; a.x must be 16-byte aligned.
hipError_t launch_qsm(const QmvArgs& a, int M, const DeviceInfo& dev);

// Few-row kernel with K split over the waves of a workgroup (2 <= M <= 16,
// 4- or 8-bit codes, group size 64 or 128, K a multiple of 512); a.x and the
// scales and biases 16-byte aligned.  K = 512 * waves * chunks with 1..8
// waves; K beyond 4096 runs in chunks (the grid's second dimension), each
// writing an f32 partial tile to the split workspace, added in a fixed order
// by the split reduction.  Chunks need f16 activations (int8 activations take
// one scale per row over all of K), M * N a multiple of 4, and a stream that
// is not being captured (`chunks_ok`).  At least one 16-row block of W per
// compute unit, counting every chunk.
bool qsmk_split(int64_t K, int* waves, int* chunks);
// The kernel's ragged variant: K not a multiple of 512, or scales / biases not
// 16-byte aligned (loaded as 2-byte values).
bool qsmk_ragged(int64_t K, const void* s, const void* b);
bool qsmk_shape(int64_t M, int64_t N, int64_t K, int bits, int group_size, bool chunks_ok, const DeviceInfo& dev);
// LDS of one workgroup; `xstage`: the activations pass through LDS first
// (f16 activations at 9..16 rows, qsmk_xstage).
size_t qsmk_lds_bytes(int waves, int bits, bool xstage);
bool qsmk_xstage(int64_t M, bool int8_act);
hipError_t launch_qsmk(const QmvArgs& a, int M, const DeviceInfo& dev);

// The split workspace cache (workspace.cpp): one f32 buffer per device and
// stream, grown on demand, at most kWorkspaceEntries streams per device (the
// least recently used is released first), shared by the prefill kernel's K
// splits and the few-row kernel's K chunks.  Hold split_workspace_mutex() from
// the call of split_workspace_locked() until the kernels that use the buffer
// are enqueued.  split_workspace_locked returns null if no memory could be had.
constexpr int kWorkspaceEntries = 4;
std::mutex& split_workspace_mutex();
float* split_workspace_locked(int device, hipStream_t stream, size_t bytes);
size_t split_workspace_cached_bytes(int device);  // takes the mutex
int split_workspace_release_all();                // takes the mutex; returns the buffers freed
// Fixed device scratch (static_scratch.hip) for the entry point that never
// allocates: kStaticScratchBytes per device, its address looked up once per
// device on first use (with that device current).
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
hipError_t static_scratch(float** out);
// y[M, N] (f16) = RNE(sum over splits of part[split] in split order + out_bias);
// M * N a multiple of 4, part 16-byte aligned.
hipError_t launch_split_reduce_f16(const float* part, const uint16_t* ob, uint16_t* y, int64_t M, int64_t N,
                                   int splits, hipStream_t stream);

struct QmmArgs {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;
  const uint16_t* ob;  // activation bits [N], added to every row of y, or null
  float* part;         // split-K workspace [splits, M, N] (set by launch_qmm)
  int splits;
  int64_t M, N, K;
  int bits;
  int group_size;
  bool sb_bf16;
  bool x_bf16;         // activations (x, y, output bias) are bf16, else f16
  hipStream_t stream;
  float* fixed_ws;        // caller-provided split workspace (no allocation), or null: the cache
  size_t fixed_ws_bytes;
};

hipError_t launch_qmm(const QmmArgs& a, const DeviceInfo& dev);
// MFMA blocks (32 x 32) per wave along M and N (the tile is (64*mb) x (64*nb))
// and the number of K splits.
struct QmmTile {
  int mb, nb, splits;
};
QmmTile qmm_pick_tile(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);
// Shapes the MFMA kernel takes: M > 8 (smaller M runs the qmv kernel), K a
// multiple of its 64-code stage, and K < 2^24 so that every per-lane offset
// within a tile (at most 128 rows of x, W, scales) fits in 32 bits.
inline bool qmm_mfma_shape(int64_t M, int64_t K) { return M > 8 && K % 64 == 0 && K < (int64_t{1} << 24); }

// int8-activation prefill kernel (qmm_a8.hip): x quantized per row once into
// a workspace, then 128 x 128 tiles on the integer matrix cores (K split when
// the tiles alone do not occupy the GPU).  Takes M >= 17, K a multiple of 64
// below 2^24 (tile-relative byte offsets fit in 32 bits), x 16-byte aligned.
inline bool qmm_a8_shape(int64_t M, int64_t K) { return M >= 17 && K % 64 == 0 && K < (int64_t{1} << 24); }
struct QmmA8Args {
  const uint16_t* x;   // f16 activations [M, K]
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;         // f16 [M, N]
  const uint16_t* ob;  // f16 [N] or null
  int64_t M, N, K;
  int bits;
  int group_size;
  bool sb_bf16;
  hipStream_t stream;
};
struct QmmA8Plan {
  int tiles_m, tiles_n, splits, nks;
  size_t part_bytes, xq_bytes, xsum_bytes, sx_bytes, workspace_bytes;
};
struct QmmA8Launch {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;
  const uint16_t* ob;
  float* part;   // [splits, M, N] f32 partial tiles, or null (one split)
  uint8_t* xq;   // [M, K] int8 activation codes
  float* xsum;   // [M, K / min(group, 64)] integer code sums
  float* sx;     // [M] row scales
  int M, N, K, tiles_m, tiles_n, splits, nks;
};
QmmA8Plan qmm_a8_plan(int64_t M, int64_t N, int64_t K, int group_size, const DeviceInfo& dev);
size_t qmm_a8_lds_bytes();
// hipErrorOutOfMemory (nothing enqueued) when no workspace can be had.
hipError_t launch_qmm_a8(const QmmA8Args& a, const DeviceInfo& dev);

// Read probe (probe.hip): streams `bytes` (a multiple of 16) from a 16-byte
// aligned buffer; out receives 4 bytes at most.
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream,
                             const DeviceInfo& dev);

struct DequantArgs {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* out;
  int64_t N, K;
  int bits;
  int glog2;
  bool sb_bf16;
  int out_dtype;  // mxq_dtype value
  hipStream_t stream;
};

hipError_t launch_dequant(const DequantArgs& a, const DeviceInfo& dev);

// y[0 .. count) = +0 (f16 bits), used for K == 0.
// y[m, n] = ob[n] (ob non-null) or +0, for m < M, n < N.
hipError_t launch_fill_rows(uint16_t* y, const uint16_t* ob, int64_t M, int64_t N, hipStream_t stream);
hipError_t launch_zero_fill(uint16_t* y, int64_t count, hipStream_t stream);

}  // namespace mxq
