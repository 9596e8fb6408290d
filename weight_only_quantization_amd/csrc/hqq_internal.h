// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hqq.h"

namespace hqq {

// Arguments of the quantizer kernels (passed by value in the kernel argument segment).
struct SolveArgs {
  const __half* W;     // [rows, cols] fp16
  uint8_t* packed;     // packed output (2/4-bit written directly)
  void* delta;         // [G] meta_dtype
  void* zero;          // [G] meta_dtype
  uint8_t* codes_ws;   // 3-bit axis 0 (and the scale search): one byte per code, packed afterwards; else nullptr
  uint32_t* edges3;    // 3-bit axis 1: per solve tile its part of the word it starts inside and of the word it
                       // ends inside ([nblocks][2]); a merge pass joins neighbours' parts
  double* partials;    // [iters][nblocks] per-block sums of |W - W_hat| per round
  int32_t* ctrl;       // [0] = index of the kept zero, [1] = rounds evaluated
  int32_t* tile_round; // [nblocks] latest round at which a wave of the tile froze (iters: one never did)
  int64_t G;           // number of groups (= M for axis 0)
  int64_t nblocks;     // blocks of the solve kernel
  int iters;
  int meta_dtype;
  double qmax;         // 2^b - 1
  double tiny;         // range at or below which s = 1
  double pm1;          // p - 1 (exponent of the shrink)
  double beta[HQQ_MAX_ITERS];        // beta_k = beta0 * kappa^k (repeated products)
  double thr[HQQ_MAX_ITERS];         // |r| below which round k's shrink is exactly 0
  double thr_frozen[HQQ_MAX_ITERS];  // min over rounds j >= k of thr[j]
};

// Quantizer: one solve pass (speculates that the loop runs all rounds), the device-side stop
// decision, a fix-up pass that redoes the groups when the loop stopped early, 3-bit packing.
// threads and lds_bytes are quant_geometry's for the configuration (the kernels assume them).
hipError_t launch_quantize(const SolveArgs& a, int nbits, int group_size, int axis, int threads, size_t lds_bytes,
                           int64_t N, int stop_rule, double* mae_trace, int32_t* stop_iter, double* reduce_ws,
                           hipStream_t stream);
// Scale search (second solver, either axis, 2/3/4-bit): the grid of multipliers of the min-max
// scale, passed by value; choice (device, optional) receives the chosen index per group.
struct ScaleGrid {
  double c[HQQ_V2_MAX_CANDIDATES];
  int n;
  uint8_t* choice;
};
// Blocks of the scale-search kernel for G groups of size g; launch (a.nblocks must be that).
int64_t quant_v2_blocks(int64_t G, int g);
hipError_t launch_quantize_v2(const SolveArgs& a, const ScaleGrid& sg, int nbits, int g, int axis, hipStream_t stream);
// Per-round entries of the intermediate levels of the stop-decision reduction.
int64_t reduce_scratch_entries(int64_t nblocks, int iters);
// Geometry of the solve kernel for a configuration: blocks, threads, dynamic LDS bytes.
bool quant_geometry(int64_t G, int group_size, int axis, int iters, int nbits, int64_t* nblocks, int* threads,
                    size_t* lds_bytes);

hipError_t launch_dequant(const uint8_t* packed, const void* delta, const void* zero, int meta_dtype,
                          int64_t rows, int64_t cols, int nbits, int group_size, int axis, __half* out,
                          hipStream_t stream);

hipError_t launch_gemv(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                       int group_size, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t stream);
size_t gemv_lds_bytes(int64_t K, int group_size, int64_t batch);

// Other stored formats (batch 1 or 2): 4-bit with axis-0 groups; 2-bit with axis-1 groups of 16.
// Split-K fused GEMM (batched product): splits of the contraction for an output length NO and a
// contraction length KC (0 = not supported), the workspace it needs (tiled A operand + fp32
// partial sums), and the launch (tiling pass, GEMM, sum).
int gemm_splits(int64_t NO, int64_t KC, int64_t batch);
size_t gemm_workspace_bytes(int64_t NO, int64_t KC, int64_t batch);
hipError_t launch_gemm_split(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                             int gs, const __half* x, int64_t batch, void* y, int y_dtype, void* workspace,
                             hipStream_t st);
// The same batched product for 2-, 3- and 4-bit codes with axis-1 groups (the staging waves
// unpack the stored format; 4-bit takes group sizes 64 and 128, 2/3-bit 16..256) and for 4-bit
// codes with axis-0 groups (axis = 0: g a power of two 16..256 dividing N).
hipError_t launch_gemm_fmt(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                           int nbits, int gs, int axis, const __half* x, int64_t batch, void* y, int y_dtype,
                           void* workspace, hipStream_t st);
// Input gradient dX [batch, K] = dY [batch, N] @ W_hat with the same kernel transposed (the
// formats of launch_gemm_fmt); its workspace is gemm_workspace_bytes(K, N, batch) (output
// length first).
hipError_t launch_gemm_dx(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          int nbits, int gs, int axis, const __half* dy, int64_t batch, void* dx, int dx_dtype,
                          void* workspace, hipStream_t st);
// Fused product at batch 1-16 on the matrix units with the tile dequantised in registers
// (2-, 3- and 4-bit codes, axis-1 groups): shapes it takes, launch.
bool gemv_dq_supported(int64_t N, int64_t K, int nbits, int g, int64_t batch);
hipError_t launch_gemv_dq(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          int nbits, int g, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st);
// Fused product with 3-bit codes (axis 1, batch 1-2): shapes it takes, LDS bytes, launch.
bool gemv_3b_supported(int64_t K, int g);
size_t gemv_3b_lds_bytes(int64_t N, int64_t K, int g, int64_t batch);
hipError_t launch_gemv_3b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                          const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st);
hipError_t launch_gemv_ax0(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                           int group_size, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t stream);
size_t gemv_ax0_lds_bytes(int64_t K, int64_t batch);
hipError_t launch_gemv_2b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t stream);
size_t gemv_2b_lds_bytes(int64_t K, int64_t batch);

hipError_t launch_gemm(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                       int group_size, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t stream);

}  // namespace hqq
