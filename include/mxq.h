/*
 * mxq.h -- C ABI of libmxq.so: matmul over affine-quantized, packed weights
 * on AMD MI355X (gfx950).
 *
 * The operation (mlxcel #574 "track(upstream-iree): fused dequant->matmul for
 * the packed int8 bandwidth win", section "What is already in-tree"; mlxcel epic
 * #570, section "Context"): weights stay resident as b-bit codes packed into
 * uint32 words plus one f16 (or bf16) scale and bias per group of `group_size`
 * codes along K; each weight is w = q * scale + bias.  The fused entry points
 * compute y = x * W^T without ever writing W to memory, which is exactly what the
 * unfused graph of epic #570 ("The measured fusion gate") fails to do.
 *
 * Layouts (all row-major, all device memory unless stated):
 *   x       f16   [M, K]            activations
 *   w       u32   [N, K*bits/32]    packed codes of W[N, K]; code k of row n is
 *                                   (w[n][k / P] >> (bits * (k % P))) & (2^bits - 1),
 *                                   P = 32 / bits (least significant field first)
 *   scales  f16|bf16 [N, K/group_size]   (sb_dtype applies to scales and biases)
 *   biases  f16|bf16 [N, K/group_size]
 *   y       f16   [M, N]            output, round-to-nearest-even of an f32 sum
 *
 * Supported: bits in {4, 8}; group_size in {32, 64, 128}; K a multiple of
 * group_size.  0 <= M, N, K < 2^31 (buffers may exceed 4 GiB); M*N == 0 is a
 * no-op that touches no pointer;
 * K == 0 with M*N > 0 writes y = +0 and reads nothing (x, w, scales and
 * biases may then be null).
 *
 * Alignment: w must be 16-byte aligned (every row then is, since a row holds
 * a multiple of four words); x, scales, biases and y must be 2-byte aligned
 * (an x that is also 16-byte aligned is staged with wider loads); the
 * dequant output `out` must be 16-byte aligned.
 *
 * Ownership and threading: every pointer is owned by the caller and must stay
 * valid until the enqueued work has finished.  The library keeps a per-device
 * cache of device properties.  It allocates device memory on three paths
 * only:
 *   - an MFMA call (mxq_qmm / mxq_linear / mxq_linear_act with M > 8 and not
 *     a few-row shape) whose 128 x 128 output tiles are too few to occupy
 *     every compute unit and whose K is long splits K: splits * M * N floats
 *     of partial results, added in a fixed order by a second kernel (16 MiB
 *     for a 512 x 2048 x 8192 call);
 *   - a few-row call (f16 activations, 2..16 rows on the K-split matrix-core
 *     kernel) with K > 4096 runs K in chunks: chunks * M * N floats;
 *   - an int8-activation call from 17 rows (mxq_linear_a8) holds the
 *     quantized activations, and, when K is split, the partial results.
 * All use one split workspace per (device, stream), from hipMalloc, grown
 * when a call needs more (the old buffer freed with hipFree, which first waits
 * for the device's enqueued work), at most 4 streams per device (the least
 * recently used stream's buffer is freed to make room), and kept until
 * mxq_release_workspaces() or the end of the process.  On a stream being
 * captured into a graph, MFMA calls allocate their workspace inside the graph
 * instead (hipMallocAsync / hipFreeAsync) and few-row calls with K > 4096 run
 * on the other kernels.  If memory cannot be had, MFMA calls run the unsplit
 * kernel, and few-row and int8 prefill calls the decode kernel.  mxq_qmm_noalloc is the variant
 * that never allocates.  Calls are thread-safe.
 *
 * Asynchrony: a call validates its arguments synchronously, enqueues its
 * kernel(s) on `stream` (a hipStream_t; NULL means the null stream) and
 * returns.  Faults inside a kernel surface at the caller's next
 * synchronisation, as for any HIP launch.  No exception crosses this ABI.
 *
 * Errors: a status other than MXQ_OK means nothing was enqueued (except
 * MXQ_ERR_HIP, returned when the launch itself failed); mxq_last_error()
 * then returns a thread-local message with the detail.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxq_status {
  MXQ_OK = 0,
  MXQ_ERR_INVALID_ARG = 1,  /* null pointer where data is needed, negative size */
  MXQ_ERR_UNSUPPORTED = 2,  /* bits, group_size, dtype, K % group_size, too-large K */
  MXQ_ERR_MISALIGNED = 3,   /* a pointer breaks the alignment rules above */
  MXQ_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} mxq_status;

typedef enum mxq_dtype {
  MXQ_F16 = 0,
  MXQ_BF16 = 1,
  MXQ_F32 = 2
} mxq_dtype;

/* Bumped whenever a signature in this header changes. */
#define MXQ_ABI_VERSION 4
int mxq_abi_version(void);

/*
 * mxq_qmv -- fused dequant + matmul tuned for decode (M = 1 .. 16).
 *
 * Computes y[m, n] = RN_f16( sum_k x[m, k] * (q[n, k] * s[n, g(k)] + b[n, g(k)]) )
 * with g(k) = k / group_size, accumulating in f32 (the scale and bias are
 * applied per group to partial sums, which is the same value up to f32
 * rounding).  The sum of epic #570's "dequant -> matmul" without the weight
 * ever leaving registers.  Accepts any M >= 0.  Routing by shape: one row
 * (and two at K > 3072) on the decode kernel; up to 16 rows on the matrix
 * cores when the shape fits them -- 4- or 8-bit codes, group size 64 or 128,
 * K at least 512 and at least 16 rows of W per compute unit (from 3 rows, or
 * 2 at K <= 3072); K beyond 4096 runs in chunks of up to 4096 codes whose f32
 * partial results are added in a fixed order by a second kernel (M * N a
 * multiple of 4, counting the chunks toward the rows of W per compute unit;
 * calls on a stream being captured into a graph use the other kernels
 * instead); K not a multiple of 512, or scales / biases only 2-byte aligned,
 * take the same kernel's ragged variant -- else 9..16 rows of any supported
 * codes with at least 256 rows of W per compute unit on a 16-row-block
 * kernel -- both with x 16-byte aligned; otherwise the decode kernel in
 * slices of at most 8 rows (each slice re-reads W).  N need not be a multiple of
 * anything (ExecuTorch PR #17187 "Description": M = 1 with N not a multiple
 * of 4).
 * Results match the f64 definition within |y - y_ref| <= 2e-3 (1 + |y_ref|)
 * and are bit-identical from run to run.
 */
mxq_status mxq_qmv(const void* x, const uint32_t* w, const void* scales, const void* biases,
                   void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                   mxq_dtype sb_dtype, void* stream);

/*
 * One problem of a grouped qmv call: y = x * dequant(w)^T with the layouts
 * above.  Pointers are device pointers; N and K are this problem's sizes.
 */
typedef struct mxq_qmv_problem {
  const void* x;          /* f16 [M, K] */
  const uint32_t* w;      /* u32 [N, K*bits/32], 16-byte aligned */
  const void* scales;     /* f16|bf16 [N, K/group_size] */
  const void* biases;     /* f16|bf16 [N, K/group_size] */
  void* y;                /* f16 [M, N] */
  int64_t N;
  int64_t K;
} mxq_qmv_problem;

/* Problems per kernel launch of mxq_qmv_grouped (larger counts use several launches). */
#define MXQ_MAX_GROUP 16

/*
 * mxq_qmv_grouped -- several independent mxq_qmv problems in one kernel launch.
 *
 * Cuts the launches per decode step (mlxcel epic #570, "The measured fusion
 * gate": ~678 dispatches per step; mlxcel #574, "Unblock criteria": the
 * dispatch count materially reduced).  All problems share M, bits, group_size
 * and sb_dtype; each has its own x, w, scales, biases, y, N and K (e.g. the
 * q, k and v projections of one layer, or gate and up).  `problems` is a host
 * array of `count` entries, read during the call only.  Results satisfy the
 * mxq_qmv contract (same tolerance, deterministic); they need not be
 * bit-identical to separate mxq_qmv calls.  Every problem is validated as in
 * mxq_qmv before anything is launched.
 */
mxq_status mxq_qmv_grouped(const mxq_qmv_problem* problems, int count, int64_t M, int bits,
                           int group_size, mxq_dtype sb_dtype, void* stream);

/*
 * mxq_qmm -- the same operation tuned for prefill (M >= 64): codes are
 * staged through LDS as exact f16 integers and contracted with f16 MFMA
 * (f32 accumulation); each group's partial products are then scaled by the
 * group's f32 scale and the bias is added as bias * sum_{k in group} x
 * (the zero-point decomposition mlxcel #574 cites in "Upstream status
 * refresh").  Same arguments, layouts, accuracy and determinism as mxq_qmv;
 * calls with M <= 8, and with up to 16 rows where the mxq_qmv matrix-core
 * route for a few rows fits, take mxq_qmv's routing.
 */
mxq_status mxq_qmm(const void* x, const uint32_t* w, const void* scales, const void* biases,
                   void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                   mxq_dtype sb_dtype, void* stream);

/*
 * mxq_qmm_noalloc -- mxq_qmm for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, and harnesses
 * that forbid allocation.  Same arguments, routing, kernels, results (bit for
 * bit) and errors as mxq_qmm, except that the f32 partial results of a split
 * or chunked K go to a fixed scratch array of 32 MiB that each GPU holds from
 * the library's load until the process ends, instead of the split workspace
 * cache: the call allocates and frees nothing (also under graph capture,
 * where it may run K in chunks).  A call that would need more than 32 MiB of
 * scratch (splits * M * N * 4 or chunks * M * N * 4 bytes) is rejected with
 * MXQ_ERR_UNSUPPORTED before anything is enqueued; mxq_last_error() names the
 * bytes needed.  The first call on a device looks up that device's scratch
 * address.  Every call on one GPU shares its scratch: calls (and replays of
 * graphs holding such calls) that may overlap in time on one GPU, on
 * different streams, race and give wrong results.  Calls ordered on one
 * stream are safe; each writes every scratch value it reads, so nothing
 * needs clearing between calls.
 */
mxq_status mxq_qmm_noalloc(const void* x, const uint32_t* w, const void* scales, const void* biases,
                           void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                           mxq_dtype sb_dtype, void* stream);

/*
 * mxq_linear -- a quantized linear layer with an output bias:
 *   y[m, n] = RNE_f16( sum_k x[m, k] * (q[n, k] * s + b) + out_bias[n] ).
 *
 * The "linear with bias" case of the 4-bit linear op whose Metal kernel
 * ExecuTorch PR #17187 ("Metal backend: import qmv_impl from MLX") imports
 * (its stack: "enable linear with bias", "test 4-bit linear with bias").
 * out_bias is an f16 device vector [N], 2-byte aligned, added in f32 before
 * the single f16 rounding; a null out_bias gives exactly the mxq_qmm result.
 * Other arguments, routing (mxq_qmv's for a few rows, MFMA kernel above),
 * accuracy and determinism as mxq_qmm; K = 0 gives y[m, n] = out_bias[n]
 * (or +0).  Errors as mxq_qmv, plus MXQ_ERR_MISALIGNED for out_bias.
 */
mxq_status mxq_linear(const void* x, const uint32_t* w, const void* scales, const void* biases,
                      const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      int group_size, mxq_dtype sb_dtype, void* stream);

/*
 * mxq_linear_act -- mxq_linear with the activation type as an argument:
 * act_dtype MXQ_F16 (the same result as mxq_linear, bit for bit) or MXQ_BF16,
 * in which case x, y and out_bias are bf16 (the other activation format of
 * MLX checkpoints).  With bf16 activations the decode kernel feeds 4-bit codes
 * to v_dot2 as bf16 integers 128 + c (exact) and takes the 128 * sum(x) back
 * through the bias term; 8-bit codes, and the codes of the MFMA kernel, are
 * converted exactly to bf16, and the MFMA kernel contracts with bf16 MFMAs.
 * Accumulation stays f32; y is the round-to-nearest-even bf16 of the f32
 * result (tolerance as mxq_qmv).  Other arguments, routing and errors as
 * mxq_linear, plus MXQ_ERR_UNSUPPORTED for another act_dtype.
 */
mxq_status mxq_linear_act(const void* x, const uint32_t* w, const void* scales, const void* biases,
                          const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                          int group_size, mxq_dtype sb_dtype, mxq_dtype act_dtype, void* stream);

/*
 * mxq_linear_a8 -- mxq_linear on the native int8 path: f16 activations are
 * quantized per row to int8 inside the kernel and contracted with the 4-bit
 * or 8-bit codes in exact integer arithmetic -- by v_dot4_i32_i8 (four
 * products per instruction) in the decode kernel, or, for 3..16 rows of
 * 4- or 8-bit codes on the shapes the K-split few-row kernel takes (group 64 or 128,
 * K a multiple of 512 up to 4096 (int8 activations are not chunked: one row
 * scale covers all of K), at least 16 rows of W per compute unit, x, scales and
 * biases 16-byte aligned), by v_mfma_i32_16x16x64_i8 (one 64-code group per
 * instruction) -- the "quantized dot lowered to the hardware's int8 path"
 * route of mlxcel #574 ("Upstream status refresh", "Next actionable step").
 * The pages define no activation scheme; the one used, dynamic per-row
 * symmetric quantization, is part of the result:
 *   amax[m] = max_k |x[m, k]|, r = 127 / amax, sx = amax / 127 (f32 quotients),
 *   xq[m, k] = clamp(rint(x[m, k] * r), -127, 127) (f32 product, ties to even),
 *   a row with amax = 0 gives xq = 0;
 *   y[m, n] = RNE_f16( sx[m] * sum_k xq[m, k] * (q[n, k] * s + b) + out_bias[n] ).
 * So y differs from mxq_linear's by the activation rounding (about 0.4 % of
 * a row's largest |x| per element); it matches the int8 method itself to the
 * tolerance of mxq_qmv.  x must be finite.
 * From 17 rows (K a multiple of 64 below 2^24, x 16-byte aligned) the call is
 * the prefill route on v_mfma_i32_32x32x32_i8: a first kernel quantizes each
 * row of x once, writing the int8 codes, the row scale and the per-group code
 * sums to a workspace (M * K + M * K / min(group, 64) * 4 + M * 4 bytes, plus
 * the f32 partial tiles when K is split, splits * M * N * 4), then 128 x 128
 * tiles read W once.  The workspace comes from the split workspace cache
 * described above (inside the graph under capture); if none can be had the
 * call takes the decode kernel instead.  Other shapes run the decode kernel
 * in slices of 8 rows.  Arguments, layouts, out_bias and errors as
 * mxq_linear.
 */
mxq_status mxq_linear_a8(const void* x, const uint32_t* w, const void* scales, const void* biases,
                         const void* out_bias, void* y, int64_t M, int64_t N, int64_t K, int bits,
                         int group_size, mxq_dtype sb_dtype, void* stream);

/*
 * mxq_dequant -- standalone dequantization: out[n, k] = q * s + b.
 *
 * The reconstruction mlxcel #574 ("What is already in-tree") requires to be
 * bit-identical to a host dequant.  out_dtype MXQ_F32 gives RN_f32(q*s + b)
 * (one rounding: q*s is exact in f32); MXQ_F16 / MXQ_BF16 give the
 * round-to-nearest-even of that f32 value (a NaN becomes 0x7FC0 in bf16).
 * `out` is [N, K] row-major, device memory.  Bit-exact by contract.
 */
mxq_status mxq_dequant(const uint32_t* w, const void* scales, const void* biases, void* out,
                       int64_t N, int64_t K, int bits, int group_size, mxq_dtype sb_dtype,
                       mxq_dtype out_dtype, void* stream);

/*
 * mxq_pack -- HOST packer for the layout above (no GPU involved).
 *
 * codes: host uint8 [N, K], each < 2^bits; w: host uint32 [N, K*bits/32]
 * written by the call.  K must be a multiple of 32/bits.  Returns
 * MXQ_ERR_INVALID_ARG if a code does not fit in `bits` bits (w is then left
 * partially written).  Synchronous.
 */
mxq_status mxq_pack(const uint8_t* codes, uint32_t* w, int64_t N, int64_t K, int bits);

/*
 * mxq_describe -- diagnostic: the kernel instantiation(s) and launch shape
 * that mxq_qmv (op "qmv"), mxq_qmm (op "qmm") or mxq_linear_a8 (op "a8")
 * would use for these sizes on the current device, e.g. "qmv_kernel<bits=4,sb=f16,mt=1,rows=4> grid=2048
 * block=256 lds=4352".  Returns a thread-local string, valid until the next
 * call on the thread; "invalid" for unsupported arguments and "no device"
 * without a GPU.  Enqueues nothing.
 */
const char* mxq_describe(const char* op, int64_t M, int64_t N, int64_t K, int bits,
                         int group_size, mxq_dtype sb_dtype);

/*
 * mxq_describe_grouped -- diagnostic: the launches mxq_qmv_grouped would make
 * for these problems on the current device (only N, K of each entry are read;
 * pointers may be null), e.g. "qmv_kernel<bits=4,sb=f16,mt=1,rows=2,xreg>
 * problems=3 grid=768 block=256 lds=0", one entry per launch separated by
 * "; ".  ",xreg" marks the variant that keeps each lane's activations in
 * registers (every K within one 64-segment step, at most two rows).  Returns
 * a thread-local string; "invalid", "none" (nothing to launch) or "no device"
 * as mxq_describe.  Enqueues nothing.
 */
const char* mxq_describe_grouped(const mxq_qmv_problem* problems, int count, int64_t M, int bits,
                                 int group_size, mxq_dtype sb_dtype);

/*
 * mxq_release_workspaces -- free every cached split workspace (see
 * "Ownership and threading" above) on every device.  Waits for each device's
 * enqueued work first (hipFree).  Later calls allocate again as needed.
 * Always MXQ_OK.
 */
mxq_status mxq_release_workspaces(void);

/* Bytes of split workspace cached for the current device (0 without a GPU). */
int64_t mxq_workspace_bytes(void);

/*
 * mxq_read_probe -- measurement aid: stream `bytes` (a multiple of 16) of
 * device memory from `buf` (16-byte aligned) with the decode kernel's load
 * form (16-byte non-temporal loads, two 256-thread workgroups per compute
 * unit) and discard the data; `out` (4 bytes of device memory, 4-byte
 * aligned) may be written with a data-dependent value.  Timing it at a size
 * gives the read bandwidth attainable at that size, against which the fused
 * kernels' figures are judged.  Errors as the fused calls.
 */
mxq_status mxq_read_probe(const void* buf, int64_t bytes, void* out, void* stream);

/* Static, human-readable name of a status. */
const char* mxq_status_str(mxq_status s);

/* Thread-local detail of the last non-OK status on this thread ("" if none). */
const char* mxq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
