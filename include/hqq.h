/*
 * hqq.h - C ABI of the HQQ weight-only quantization library for AMD Instinct
 * MI355X (gfx950).
 *
 * HQQ (half-quadratic quantization) is a calibration-free, group-wise,
 * asymmetric affine weight quantizer.  The operations below follow the page
 * "HQQ 算法解读：不用校准数据，怎样把大模型权重压到 4 bit"
 * (ludovicoyin.github.io/blog/posts/hqq-half-quadratic-quantization):
 *   - "量化公式": q = clip(round(W*s + z), 0, 2^b-1), W_hat = (q - z) * delta,
 *     delta = 1/s is the stored step ("scale"), z the zero in code units;
 *   - "第一拍": min-max start s0 = (2^b-1)/(max-min), z0 = -min*s0, s = 1 when the
 *     range is tiny, s limited to at most 2e4;
 *   - "第二拍" and "为什么 zero 是这个均值": up to `iters` proximal rounds that move
 *     only the zero, z <- mean(q - (W - e)*s) with e = shrink(W - W_hat) (lp
 *     shrink, p, beta growing by kappa per round), stopping when the
 *     whole-tensor reconstruction MAE no longer improves and going back to the
 *     zero that reached the best MAE; then one final quantisation of W;
 *   - "为什么一定要分组": bit-packing, two 4-bit codes per byte, four 2-bit codes
 *     per byte, ten 3-bit codes per 32-bit word;
 *   - "axis 不是一个无关紧要的开关": groups are reshape([-1, g]) rows (axis=1) or
 *     reshape([g, -1]) columns (axis=0) of the row-major [rows, cols] weight;
 *   - "从压缩文件到一次前向": unpack, (q - zero) * scale, x @ W_hat^T.
 *
 * Shrink reading (the page names the operator but prints no formula):
 *   e = sign(r) * max(|r| - |r|^(p-1) / beta, 0), e = 0 at r = 0.
 * Stop reading: round k's MAE measures z_k; the loop stops at the first k >= 1
 * whose MAE is not below the best so far, and keeps z_(k-1); when no round
 * stops it, z_iters (the last update) is kept.
 *
 * Data layout (all buffers are device memory, caller-owned):
 *   W          fp16 [rows, cols], row-major.
 *   packed     codes in flat row-major order (the same order for both axes),
 *              little-endian inside each container:
 *                4-bit: byte j = c[2j] | c[2j+1] << 4            (rows*cols/2 bytes)
 *                2-bit: byte j = sum_t c[4j+t] << 2t             (rows*cols/4 bytes)
 *                3-bit: uint32 j = sum_t c[10j+t] << 3t, bits 30-31 zero, the last
 *                       word padded with code 0          (4*ceil(rows*cols/10) bytes)
 *   delta/zero one value per group, group j in the order of the group view:
 *                axis=1: group j = flat elements j*g .. j*g+g-1  ([rows, cols/g]);
 *                axis=0: group j = flat elements i*(N/g) + j     ([rows/g, cols]).
 *
 * Conventions:
 *   - Ownership: every pointer is caller-owned device memory (workspace
 *     included).  The library allocates, frees and retains nothing (its only device
 *     memory is the static scratch array of hqq_quantize_noalloc).
 *   - Asynchrony: every compute call only enqueues work on `stream` (a
 *     hipStream_t, NULL = the default stream) and returns; nothing is
 *     synchronised.  Outputs are valid once the stream has reached that point.
 *   - Alignment: W, packed, delta, zero, x, y and the workspace must be 16-byte
 *     aligned (torch allocations are 256-byte aligned).
 *   - Inputs are read only; outputs are fully overwritten; inputs and outputs
 *     must not overlap.  Inputs must be finite.
 *   - Errors: arguments are checked before anything is enqueued; a non-zero
 *     status means nothing was launched (HQQ_ERR_DEVICE: a launch failed; the
 *     message is in hqq_last_error()).  No exception crosses the ABI.
 *   - State: the library keeps no mutable global state, so calls on different
 *     streams may run concurrently (with distinct workspaces); the one exception is
 *     hqq_quantize_noalloc, whose calls on one GPU share that GPU's scratch array.
 */
#ifndef HQQ_H
#define HQQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define HQQ_OK 0
#define HQQ_ERR_INVALID_ARGUMENT 1 /* a pointer, size or parameter is outside the contract */
#define HQQ_ERR_UNSUPPORTED 2      /* valid HQQ, but a shape/format the library has no kernel for */
#define HQQ_ERR_WORKSPACE 3        /* workspace missing or smaller than hqq_quantize_workspace_bytes */
#define HQQ_ERR_DEVICE 4           /* a HIP call or kernel launch failed */

/* Metadata element types (delta and zero share one type). */
#define HQQ_META_F16 0 /* the stored format: fp16 scale + fp16 zero, 4.5 bits/weight at 4-bit g64 */
#define HQQ_META_F32 1
#define HQQ_META_F64 2 /* the solver's own precision (quantize only) */

/* GEMV / GEMM output types. */
#define HQQ_OUT_F16 0
#define HQQ_OUT_F32 1

/* Range max-min at or below which s = 1 ("第一拍" sets s = 1 for a tiny range but
 * gives no threshold; this library uses 1e-4). */
#define HQQ_TINY_RANGE 1e-4
/* s is limited to at most this value ("第一拍"). */
#define HQQ_MAX_SCALE 2.0e4
/* Largest accepted `iters`. */
#define HQQ_MAX_ITERS 64
/* Multipliers of the scale search (hqq_quantize_v2) at most. */
#define HQQ_V2_MAX_CANDIDATES 16

/* Bytes of the packed code buffer for rows*cols codes of `nbits` (2, 3 or 4), or 0
 * when the arguments are invalid. */
size_t hqq_packed_bytes(int64_t rows, int64_t cols, int nbits);

/* Number of groups rows*cols/group_size, or -1 when group_size does not divide it. */
int64_t hqq_num_groups(int64_t rows, int64_t cols, int group_size);

/* Workspace bytes hqq_quantize needs for these arguments, or 0 when they are invalid. */
size_t hqq_quantize_workspace_bytes(int64_t rows, int64_t cols, int nbits, int group_size, int axis, int iters);

/*
 * HQQ quantisation of one weight tensor ("第一拍", "第二拍", "为什么一定要分组").
 *   W_fp16     in   fp16 [rows, cols] row-major.
 *   nbits      2, 3 or 4.
 *   group_size 16, 32, 64, 128 or 256; it must divide cols (axis=1) or rows (axis=0);
 *              axis=0 also needs (rows/group_size)*cols to be a multiple of 8.
 *   axis       1 (groups along a row) or 0 (groups down a column, row stride rows/g).
 *   iters      0 .. HQQ_MAX_ITERS proximal rounds at most (20 on the page).
 *   p          lp exponent of the shrink, 0 < p <= 1 (0.7 on the page).
 *   beta0      shrink beta of round 0, > 0 (10 on the page).
 *   kappa      beta growth per round, > 0 (1.01 on the page).
 *   packed     out  hqq_packed_bytes(rows, cols, nbits) bytes.
 *   delta      out  one step (1/s) per group, type meta_dtype.
 *   zero       out  one zero per group (code units), type meta_dtype.
 *   meta_dtype HQQ_META_F16, HQQ_META_F32 or HQQ_META_F64; values are rounded to
 *              nearest-even from the solver's fp64 values.
 *   workspace  device scratch of at least hqq_quantize_workspace_bytes(...) bytes;
 *              its contents on entry do not matter.
 *   stop_iter_dev  out (nullable) device int32: index k_out of the kept zero
 *              (iters when the loop ran to the end).
 *   mae_trace_dev  out (nullable) device double[iters]: the whole-tensor MAE of each
 *              round the method evaluates; entries past the stop are NaN.
 *   stream     hipStream_t or NULL.
 * The solver runs in fp64 on the GPU; the stop decision stays on the device (no
 * host round trip).
 */
int hqq_quantize(const void* W_fp16, int64_t rows, int64_t cols, int nbits, int group_size, int axis, int iters,
                 double p, double beta0, double kappa, void* packed, void* delta, void* zero, int meta_dtype,
                 void* workspace, size_t workspace_bytes, int32_t* stop_iter_dev, double* mae_trace_dev,
                 void* stream);

/*
 * Allocation-free variant of hqq_quantize, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * operation, arguments (without the workspace), layout, ownership of the caller's buffers and
 * asynchrony as hqq_quantize; its workspace is a device array owned by the library, one copy per
 * GPU of HQQ_NOALLOC_SCRATCH_BYTES, set up on the first call on that device (with the device
 * current) and held until the process ends.  It calls no hipMalloc, hipFree or allocating
 * library routine.  Limit: tensors whose hqq_quantize_workspace_bytes(...) exceeds
 * HQQ_NOALLOC_SCRATCH_BYTES are refused with HQQ_ERR_WORKSPACE before anything is enqueued
 * (e.g. the per-round error sums of 20 rounds over a 28672x8192 tensor take 19 MB; 3-bit codes
 * with axis-0 groups take one more byte per weight).  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be serialised by the caller;
 * the array needs no clearing between calls (no part of it has to start at zero).
 */
#define HQQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int hqq_quantize_noalloc(const void* W_fp16, int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                         int iters, double p, double beta0, double kappa, void* packed, void* delta, void* zero,
                         int meta_dtype, int32_t* stop_iter_dev, double* mae_trace_dev, void* stream);

/* Stop rules of hqq_quantize_ex: readings of "第二拍" (the loop stops at the first round k >= 1
 * whose whole-tensor MAE is not below the best so far, and rolls back to the previous
 * parameters; the page gives no result for a loop that never stops).  hqq_quantize uses 0. */
#define HQQ_STOP_BEST 0         /* keep z_(k-1), the zero of the best round */
#define HQQ_STOP_FAILED 1       /* keep z_k, the zero the failing round used */
#define HQQ_STOP_NONE 2         /* keep z_(k+1), the update the failing round computed */
#define HQQ_STOP_MEASURED_END 4 /* flag: a loop that never stops keeps z_(iters-1), the last zero
                                   whose error was measured, instead of z_iters */
/* Debug flags of hqq_quantize_ex.  The first two switch off exact shortcuts of the solver,
 * so the results do not change; they exist to show that. */
#define HQQ_DEBUG_NO_FROZEN_SKIP 1 /* run every round of every group (no fixed-point skip) */
#define HQQ_DEBUG_SLOW_SHRINK 2    /* evaluate the shrink for every residual (no zero fast path) */
#define HQQ_DEBUG_SYNC 4           /* wait for the stream after the launches and report a kernel
                                      failure as HQQ_ERR_DEVICE (the call then blocks) */

/* Arguments of hqq_quantize_ex: those of hqq_quantize, then the stop rule, the tiny-range
 * threshold of the start (s = 1 when max - min <= tiny_range; >= 0, hqq_quantize uses
 * HQQ_TINY_RANGE) and the debug flags. */
typedef struct hqq_quant_args {
  const void* W_fp16;
  int64_t rows, cols;
  int nbits, group_size, axis, iters;
  double p, beta0, kappa;
  void* packed;
  void* delta;
  void* zero;
  int meta_dtype;
  void* workspace;
  size_t workspace_bytes;
  int32_t* stop_iter_dev;
  double* mae_trace_dev;
  void* stream;
  int stop_rule;
  double tiny_range;
  int debug_flags;
} hqq_quant_args;

/*
 * hqq_quantize with the choices the page leaves open ("第一拍": the tiny-range threshold;
 * "第二拍": which zero the stop keeps) and debug flags.  Same buffers, layout, ownership and
 * asynchrony as hqq_quantize (except HQQ_DEBUG_SYNC); stop_iter_dev receives the index of
 * the kept zero under the chosen rule.  Returns HQQ_ERR_INVALID_ARGUMENT for a NULL args, a
 * stop_rule outside {0, 1, 2, 4, 5, 6}, a negative or non-finite tiny_range or unknown flags.
 */
int hqq_quantize_ex(const hqq_quant_args* args);

/*
 * Scale search: the slower second solver of the method ("第二拍" names it next to the default
 * one, which keeps the min-max scale and only refines the zero; this one can grid-search the
 * scale).  The page gives its name and purpose only; the reading implemented (and its oracle)
 * is: for each group and each multiplier c_j of scale_grid, s = min(s0 * c_j, 2e4) with s0 the
 * min-max start before its limit, delta = 1/s, z0 = -min * s, up to `iters` proximal rounds
 * (shrink p, beta_k = beta0 * kappa^k) stopped by the default rule applied to the group's own
 * error sum (keep z_(k-1) at the first k >= 1 whose sum is not below the previous one, else
 * z_iters), and the group's sum of |W - W_hat| over its final codes; the first candidate with
 * the smallest sum wins.  There is no whole-tensor stop and no workspace.
 *
 * Arguments as hqq_quant_args where named alike (either axis, with hqq_quantize's shape
 * rules); scale_grid is a HOST array of n_candidates (1 .. HQQ_V2_MAX_CANDIDATES)
 * finite positive multipliers, read before the call returns; choice_dev (device, may be NULL)
 * receives the chosen index per group (G bytes); workspace (device, 16-byte aligned) holds
 * hqq_quantize_v2_workspace_bytes(rows, cols, nbits) bytes (the 3-bit codes before packing; 0
 * for 2 and 4 bits, when it may be NULL; HQQ_ERR_WORKSPACE if smaller).  Outputs: packed
 * codes, delta and zero (meta_dtype) as hqq_quantize.  Validation errors return before any
 * launch; the work is enqueued on `stream` and is asynchronous.
 */
typedef struct hqq_quant_v2_args {
  const void* W_fp16;
  int64_t rows, cols;
  int nbits, group_size, axis, iters;
  double p, beta0, kappa, tiny_range;
  const double* scale_grid;
  int n_candidates;
  void* packed;
  void* delta;
  void* zero;
  int meta_dtype;
  uint8_t* choice_dev;
  void* stream;
  void* workspace;
  size_t workspace_bytes;
} hqq_quant_v2_args;

size_t hqq_quantize_v2_workspace_bytes(int64_t rows, int64_t cols, int nbits);
int hqq_quantize_v2(const hqq_quant_v2_args* args);

/*
 * Standalone dequantisation ("量化公式", "从压缩文件到一次前向"):
 * W_out[i] = fp16((q_i - zero[j]) * delta[j]), j the group of flat element i.
 *   packed, delta, zero  in  the buffers hqq_quantize wrote (same rows, cols, nbits,
 *                        group_size, axis); meta_dtype HQQ_META_F16 or HQQ_META_F32.
 *   W_out_fp16           out fp16 [rows, cols] row-major.
 * The product is formed exactly and rounded once to nearest-even fp16.  With fp16
 * metadata this holds for every value (a zero result is +0 where a step <= 0 would
 * give -0; quantizer steps are positive); with fp32 metadata the difference q - z
 * may carry one fp32 rounding when 0 < |zero| < 2^-10.
 */
int hqq_dequantize(const void* packed, const void* delta, const void* zero, int meta_dtype, int64_t rows,
                   int64_t cols, int nbits, int group_size, int axis, void* W_out_fp16, void* stream);

/*
 * Fused dequantise + matrix product with 4-bit weights and fp16 activations
 * ("从压缩文件到一次前向": y = x @ W_hat^T, W_hat = (q - zero) * scale):
 *   y[b, n] = sum_k x[b, k] * (q[n, k] - zero[n, k/g]) * delta[n, k/g].
 *   packed      in  4-bit codes of W [N, K] (axis=1 groups along K).
 *   delta_fp16, zero_fp16  in  fp16 [N, K/group_size].
 *   group_size  64 or 128.
 *   x_fp16      in  fp16 [batch, K] row-major.
 *   y           out [batch, N] row-major, y_dtype HQQ_OUT_F16 or HQQ_OUT_F32.
 * N must be a multiple of 16 and K of 128.  Kernels by batch and size (fp32 accumulation in
 * all; each deterministic):
 *   batch 1-2: a streaming kernel that keeps q exact and applies delta and zero per group on
 *     fp32 partial sums (the MFMA GEMV below for rows longer than 16384 codes);
 *   batch 3-8 with N * K <= 2^24, and batch 9-16 with N * K <= 2^26 (K <= 32768): codes
 *     dequantised to fp16 W_hat = fp16(q delta - z delta) (exact value, rounded once) in
 *     registers, multiplied on the MFMA unit, K split over a block's waves;
 *   batch 3-8 otherwise: an MFMA GEMV that keeps q exact, the packed rows staged in LDS;
 *   above that, MFMA GEMMs on fp16 W_hat tiles.
 * Above batch 8 (past the sizes above), with N a multiple of 128 and K of 256, the call runs
 * the split GEMM of hqq_gemm_w4a16 on a workspace the library owns: one device buffer per
 * (device, stream), allocated (hipMalloc, after synchronising that stream when an older,
 * smaller one is replaced) on the first call that needs more than the stream's buffer holds,
 * and kept until hqq_release_workspaces or the end of the process.  Calls on different streams never share
 * a buffer.  Callers that must not allocate (inside graph capture, say) make one call of the
 * largest batch on the stream first, or call hqq_gemm_w4a16 with their own workspace.  Other
 * shapes above batch 8 run a single-pass MFMA GEMM with no workspace.
 */
int hqq_gemv_w4a16(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                   int group_size, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* stream);

/*
 * Frees the workspaces hqq_gemv_w4a16 keeps per (device, stream) (waits for each device's
 * work).  The next call that runs the split GEMM allocates again.  No call of hqq_gemv_w4a16
 * may run concurrently on another host thread.  Returns HQQ_OK or HQQ_ERR_DEVICE.
 */
int hqq_release_workspaces(void);

/*
 * Batched fused product with a caller-provided workspace (same operation, operands and
 * output layout as hqq_gemv_w4a16; "从压缩文件到一次前向": y = x @ W_hat^T).  For large
 * batches: each block of the GPU computes a 256 (batch) x 128 (weight rows) tile over a
 * share of K, the weight tile dequantised once into LDS, fp16 MFMA with fp32 accumulation;
 * the K shares' fp32 partial sums are added in a fixed order (deterministic).
 *   workspace        device memory of at least hqq_gemm_workspace_bytes(N, K, batch) bytes,
 *                    16-byte aligned, owned by the caller; overwritten (a tiled copy of x and
 *                    the partial sums); calls that share a workspace must not overlap.
 * N must be a multiple of 128 and K of 256; group_size 64 or 128; any batch >= 1 (rows are
 * processed in blocks of 256).  Returns HQQ_ERR_UNSUPPORTED for other shapes and
 * HQQ_ERR_WORKSPACE when the workspace is too small.
 */
size_t hqq_gemm_workspace_bytes(int64_t N, int64_t K, int64_t batch);
int hqq_gemm_w4a16(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                   int group_size, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The batched product for the other stored formats ("为什么一定要分组" for the containers,
 * "从压缩文件到一次前向" for the product, "`axis` 不是一个无关紧要的开关" for axis 0):
 * y = x @ W_hat^T as hqq_gemm_w4a16, for codes of nbits = 2, 3 or 4 with axis-1 groups and
 * 4-bit codes with axis-0 groups, stored as hqq_quantize wrote them.
 *   packed, delta_fp16, zero_fp16, N, K, nbits, group_size, axis  as hqq_gemv.
 *   x_fp16, batch, y, y_dtype  as hqq_gemm_w4a16.
 *   workspace   at least hqq_gemm_workspace_bytes(N, K, batch) bytes, as hqq_gemm_w4a16.
 * The same split MFMA kernel: only the weight tile's staging depends on the format (ten
 * 3-bit codes per word, rows starting inside words; four 2-bit codes per byte; axis 0: each
 * code with the step and zero of metadata row n mod (N/g) at its column).  N a multiple of
 * 128, K of 256; group_size 64 or 128 for 4-bit axis-1 codes (the hqq_gemm_w4a16 path), a
 * power of two 16..256 for 2/3-bit and axis-0 codes; 2/3-bit codes with axis 0 and other
 * shapes return HQQ_ERR_UNSUPPORTED.  Any batch >= 1 (batches up to 16 for 3/2-bit codes, or 8
 * for axis-0 codes, are cheaper through hqq_gemv).
 */
int hqq_gemm(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
             int group_size, int axis, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * Input gradient of the fused product, for training through frozen quantised weights
 * ("从压缩文件到一次前向": the forward is y = x @ W_hat^T, so dL/dx = dL/dy @ W_hat):
 *   dX[b, k] = sum_n dY[b, n] * (q[n, k] - zero[n, k/g]) * delta[n, k/g].
 *   packed, delta_fp16, zero_fp16, group_size  as hqq_gemm_w4a16 (W [N, K], 4-bit, axis 1).
 *   dy_fp16     in  fp16 [batch, N] row-major.
 *   dx          out [batch, K] row-major, dx_dtype HQQ_OUT_F16 or HQQ_OUT_F32.
 *   workspace   at least hqq_gemm_dx_workspace_bytes(N, K, batch) bytes, as hqq_gemm_w4a16.
 * The same split MFMA kernel with the weight tile transposed in LDS (the packed format is read
 * as stored); fp32 accumulation, splits of N added in a fixed order.  K must be a multiple of
 * 128 and N of 256; other shapes return HQQ_ERR_UNSUPPORTED.
 */
size_t hqq_gemm_dx_workspace_bytes(int64_t N, int64_t K, int64_t batch);
int hqq_gemm_w4a16_dx(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                      int group_size, const void* dy_fp16, int64_t batch, void* dx, int dx_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The input gradient for the other stored formats ("从压缩文件到一次前向" for the product,
 * "为什么一定要分组" for the containers): dX = dY @ W_hat as hqq_gemm_w4a16_dx, for the formats
 * of hqq_gemm (2-, 3- and 4-bit codes with axis-1 groups, 4-bit codes with axis-0 groups).
 *   packed, delta_fp16, zero_fp16, N, K, nbits, group_size, axis  as hqq_gemm.
 *   dy_fp16, batch, dx, dx_dtype  as hqq_gemm_w4a16_dx.
 *   workspace   at least hqq_gemm_dx_workspace_bytes(N, K, batch) bytes, as hqq_gemm_w4a16.
 * The transposed split kernel: each staging thread unpacks 32 codes of two weight rows (ten
 * 3-bit codes per word, four 2-bit codes per byte) and writes them column-major into the LDS
 * tile.  K a multiple of 128, N of 256; group sizes as hqq_gemm; 2/3-bit codes with axis 0
 * and other shapes return HQQ_ERR_UNSUPPORTED.
 */
int hqq_gemm_dx(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
                int group_size, int axis, const void* dy_fp16, int64_t batch, void* dx, int dx_dtype, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * The same fused product for the other stored formats ("从压缩文件到一次前向";
 * "axis 不是一个无关紧要的开关" for axis 0; "为什么一定要分组" for the containers):
 *   y[b, n] = sum_k x[b, k] * (q[n, k] - zero[j]) * delta[j],  j the group of code (n, k)
 *   in the group view of W [N, K] (axis=1: j = (n*K + k)/g; axis=0: j = (n*K + k) mod (N*K/g),
 *   i.e. metadata row n mod (N/g), column k).
 *   packed      in  codes of W [N, K] as hqq_quantize wrote them (nbits, group_size, axis).
 *   delta_fp16, zero_fp16  in  fp16, one per group in group-view order.
 *   x_fp16      in  fp16 [batch, K];  y out [batch, N], y_dtype HQQ_OUT_F16 or HQQ_OUT_F32.
 * Supported: nbits=4 axis=1 (as hqq_gemv_w4a16); nbits=4 axis=0 with group_size 16..256,
 * K a multiple of 32, batch 1 or 2, K <= 16384, or batch 3..8 with K a multiple of 128 (the
 * MFMA unit; any K); nbits=2 axis=1 group_size 16 with N a multiple of 16, K a multiple of
 * 64, batch 1 or 2, K <= 16384; nbits=3 axis=1 with group_size 16..256, N a multiple of 4,
 * 40 <= K <= 8192, batch 1 or 2 (rows start inside the ten-code words); nbits=3 (group_size
 * 16..256) and nbits=2 (group_size 16) axis=1 at batch 3..16 with any N and K a multiple of
 * 128, K <= 12288 (3-bit) or 16384 (2-bit), twice that with at most 8160 rows.  Other
 * combinations return HQQ_ERR_UNSUPPORTED.  Batches 1-2 and axis-0 codes keep the codes exact
 * (fp16 subnormals into v_dot2_f32_f16 or v_mfma_f32_16x16x32_f16; axis 0 forms
 * a = x * delta of the weight's metadata row in fp16, one rounding, and subtracts sum_k a z);
 * 3/2-bit batches 3..16 dequantise each code to fp16 W_hat = fp16(q delta - z delta) (one
 * rounding of the exact value) in registers and multiply on v_mfma_f32_16x16x32_f16.  fp32
 * sums throughout; the waves' partial sums are added in a fixed order (deterministic).
 */
int hqq_gemv(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
             int group_size, int axis, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* stream);

/* Static description of a status code. */
const char* hqq_status_string(int status);

/* Message of the last HQQ_ERR_* returned on the calling thread ("" if none). */
const char* hqq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HQQ_H */
