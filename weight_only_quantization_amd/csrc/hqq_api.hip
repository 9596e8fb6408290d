// C ABI of the HQQ library: argument checks, workspace layout, kernel dispatch.
// Every check happens before anything is enqueued; no exception crosses the boundary.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <thread>
#include <vector>

#include "hqq_internal.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int device_fail(hipError_t e, const char* what) {
  return fail(HQQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_group(int g) { return g == 16 || g == 32 || g == 64 || g == 128 || g == 256; }

// Shared shape checks of quantize / dequantize.  Returns HQQ_OK or an error (message set).
int check_shape(int64_t rows, int64_t cols, int nbits, int g, int axis) {
  if (rows <= 0 || cols <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "rows and cols must be positive");
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31) || rows * cols > (int64_t(1) << 40))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "tensor too large");
  if (nbits != 2 && nbits != 3 && nbits != 4) return fail(HQQ_ERR_INVALID_ARGUMENT, "nbits must be 2, 3 or 4");
  if (axis != 0 && axis != 1) return fail(HQQ_ERR_INVALID_ARGUMENT, "axis must be 0 or 1");
  if (g <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must be positive");
  if ((axis == 1 ? cols : rows) % g != 0)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size %d does not divide %s", g, axis == 1 ? "cols" : "rows");
  if (!pow2_group(g)) return fail(HQQ_ERR_UNSUPPORTED, "group_size must be 16, 32, 64, 128 or 256");
  if (axis == 0 && ((rows / g) * cols) % 8 != 0)
    return fail(HQQ_ERR_UNSUPPORTED, "axis=0 needs (rows/group_size)*cols to be a multiple of 8");
  return HQQ_OK;
}

struct QuantLayout {
  int64_t G, nblocks;
  int threads;
  size_t lds;
  size_t off_partials, off_reduce, off_rounds, off_codes, total;
};

bool quant_layout(int64_t rows, int64_t cols, int nbits, int g, int axis, int iters, QuantLayout* q) {
  q->G = rows * cols / g;
  if (!hqq::quant_geometry(q->G, g, axis, iters, nbits, &q->nblocks, &q->threads, &q->lds)) return false;
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  q->off_partials = 256;
  q->off_reduce = up(q->off_partials + (size_t)iters * q->nblocks * sizeof(double));
  q->off_rounds = up(q->off_reduce + (size_t)iters * hqq::reduce_scratch_entries(q->nblocks, iters) * sizeof(double));
  q->off_codes = up(q->off_rounds + (size_t)q->nblocks * sizeof(int32_t));
  // 3-bit codes: axis 1 packs them in the solve (two partial words per tile for the words shared
  // with a neighbouring tile); axis 0 keeps one byte per code for the packing pass
  q->total = q->off_codes + (nbits == 3 ? (axis == 1 ? up((size_t)q->nblocks * 2 * sizeof(uint32_t))
                                                     : up((size_t)(rows * cols)))
                                        : 0);
  return true;
}

}  // namespace

extern "C" {

size_t hqq_packed_bytes(int64_t rows, int64_t cols, int nbits) {
  if (rows <= 0 || cols <= 0) return 0;
  const int64_t N = rows * cols;
  if (nbits == 4) return (size_t)((N + 1) / 2);
  if (nbits == 2) return (size_t)((N + 3) / 4);
  if (nbits == 3) return (size_t)(4 * ((N + 9) / 10));
  return 0;
}

int64_t hqq_num_groups(int64_t rows, int64_t cols, int group_size) {
  if (rows <= 0 || cols <= 0 || group_size <= 0) return -1;
  const int64_t N = rows * cols;
  return N % group_size == 0 ? N / group_size : -1;
}

size_t hqq_quantize_workspace_bytes(int64_t rows, int64_t cols, int nbits, int group_size, int axis, int iters) {
  if (check_shape(rows, cols, nbits, group_size, axis) != HQQ_OK || iters < 0 || iters > HQQ_MAX_ITERS) return 0;
  QuantLayout q;
  if (!quant_layout(rows, cols, nbits, group_size, axis, iters, &q)) return 0;
  return q.total;
}

}  // extern "C"

namespace {

// hqq_quantize and hqq_quantize_ex: validation, the solver's per-round constants, the launches.
// beta_k by repeated products (beta grows by kappa after every round); thresholds of the
// shrink: e = 0 exactly for |r| <= beta^(-1/(2-p)); a 1e-6 relative margin keeps the fast
// path strictly inside that region.
void fill_schedule(hqq::SolveArgs& a, int iters, double p, double beta0, double kappa) {
  double beta = beta0;
  for (int k = 0; k < iters; ++k) {
    a.beta[k] = beta;
    a.thr[k] = pow(beta, -1.0 / (2.0 - p)) * (1.0 - 1e-6);
    beta = beta * kappa;
  }
}

int quantize_impl(const hqq_quant_args& x) {
  const void* W_fp16 = x.W_fp16;
  const int64_t rows = x.rows, cols = x.cols;
  const int nbits = x.nbits, group_size = x.group_size, axis = x.axis, iters = x.iters, meta_dtype = x.meta_dtype;
  const double p = x.p, beta0 = x.beta0, kappa = x.kappa;
  void *packed = x.packed, *delta = x.delta, *zero = x.zero, *workspace = x.workspace;
  const size_t workspace_bytes = x.workspace_bytes;
  int32_t* stop_iter_dev = x.stop_iter_dev;
  double* mae_trace_dev = x.mae_trace_dev;
  int st = check_shape(rows, cols, nbits, group_size, axis);
  if (st != HQQ_OK) return st;
  if (iters < 0 || iters > HQQ_MAX_ITERS) return fail(HQQ_ERR_INVALID_ARGUMENT, "iters must be in [0, %d]", HQQ_MAX_ITERS);
  if (!(p > 0.0 && p <= 1.0)) return fail(HQQ_ERR_INVALID_ARGUMENT, "p must be in (0, 1]");
  if (!(beta0 > 0.0) || !isfinite(beta0)) return fail(HQQ_ERR_INVALID_ARGUMENT, "beta0 must be positive");
  if (!(kappa > 0.0) || !isfinite(kappa)) return fail(HQQ_ERR_INVALID_ARGUMENT, "kappa must be positive");
  if (meta_dtype != HQQ_META_F16 && meta_dtype != HQQ_META_F32 && meta_dtype != HQQ_META_F64)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "meta_dtype must be HQQ_META_F16, _F32 or _F64");
  if (!W_fp16 || !packed || !delta || !zero) return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(W_fp16) || !aligned16(packed) || !aligned16(delta) || !aligned16(zero))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(stop_iter_dev) & 3u) || (reinterpret_cast<uintptr_t>(mae_trace_dev) & 7u))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "stop_iter_dev / mae_trace_dev misaligned");
  QuantLayout q;
  if (!quant_layout(rows, cols, nbits, group_size, axis, iters, &q))
    return fail(HQQ_ERR_UNSUPPORTED, "configuration needs more LDS than one block may use");
  if (!workspace || workspace_bytes < q.total)
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes needed", q.total);
  if (!aligned16(workspace)) return fail(HQQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  hqq::SolveArgs a;
  memset(&a, 0, sizeof(a));
  a.W = reinterpret_cast<const __half*>(W_fp16);
  a.packed = reinterpret_cast<uint8_t*>(packed);
  a.delta = delta;
  a.zero = zero;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  a.ctrl = reinterpret_cast<int32_t*>(ws);
  a.partials = reinterpret_cast<double*>(ws + q.off_partials);
  a.tile_round = reinterpret_cast<int32_t*>(ws + q.off_rounds);
  a.codes_ws = (nbits == 3 && axis == 0) ? ws + q.off_codes : nullptr;
  a.edges3 = (nbits == 3 && axis == 1) ? reinterpret_cast<uint32_t*>(ws + q.off_codes) : nullptr;
  a.G = q.G;
  a.nblocks = q.nblocks;
  a.iters = iters;
  a.meta_dtype = meta_dtype;
  a.qmax = (double)((1 << nbits) - 1);
  a.tiny = x.tiny_range;
  a.pm1 = p - 1.0;
  fill_schedule(a, iters, p, beta0, kappa);
  double m = INFINITY;
  for (int k = iters - 1; k >= 0; --k) {
    m = fmin(m, a.thr[k]);
    a.thr_frozen[k] = (x.debug_flags & HQQ_DEBUG_NO_FROZEN_SKIP) ? -1.0 : m;  // -1: no group ever freezes
    if (x.debug_flags & HQQ_DEBUG_SLOW_SHRINK) a.thr[k] = 0.0;               // every residual takes pow()
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(x.stream);
  hipError_t e = hqq::launch_quantize(a, nbits, group_size, axis, q.threads, q.lds, rows * cols, x.stop_rule,
                                      mae_trace_dev, stop_iter_dev, reinterpret_cast<double*>(ws + q.off_reduce),
                                      hs);
  if (e != hipSuccess) return device_fail(e, "hqq_quantize launch");
  if (x.debug_flags & HQQ_DEBUG_SYNC) {
    e = hipStreamSynchronize(hs);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return device_fail(e, "hqq_quantize kernels");
  }
  return HQQ_OK;
}

}  // namespace

extern "C" {

int hqq_quantize(const void* W_fp16, int64_t rows, int64_t cols, int nbits, int group_size, int axis, int iters,
                 double p, double beta0, double kappa, void* packed, void* delta, void* zero, int meta_dtype,
                 void* workspace, size_t workspace_bytes, int32_t* stop_iter_dev, double* mae_trace_dev,
                 void* stream) {
  g_last_error[0] = 0;
  const hqq_quant_args x = {W_fp16, rows, cols, nbits, group_size, axis, iters, p, beta0, kappa, packed, delta,
                            zero, meta_dtype, workspace, workspace_bytes, stop_iter_dev, mae_trace_dev, stream,
                            HQQ_STOP_BEST, HQQ_TINY_RANGE, 0};
  return quantize_impl(x);
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// Allocation-free quantisation: the workspace of hqq_quantize in a library-owned device array
// (one copy per GPU, held until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken per device with
// hipGetSymbolAddress on the first call there and only that address is handed to kernels.
// ------------------------------------------------------------------------------------------
namespace {

static __device__ __align__(256) uint8_t scratch[HQQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (set up once per device, with it current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HQQ_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned16(ptr)) return fail(HQQ_ERR_DEVICE, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HQQ_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Library-owned workspaces of hqq_gemv_w4a16 above batch 8 (the split GEMM needs a tiled copy
// of x and the splits' partial sums): one buffer per (device, stream), grown on demand and kept
// until hqq_release_workspaces or the end of the process.  Calls on one stream run in order and
// share its buffer; calls on different streams never share one (hipStreamPerThread is a
// different stream on every host thread, so its entries are per thread).  g_ws_mutex is held
// while a call enqueues its kernels, so calls from several host threads on one stream do not
// interleave on the buffer.
// ------------------------------------------------------------------------------------------
namespace {

struct StreamWs {
  int dev;
  hipStream_t st;
  std::thread::id thread;  // hipStreamPerThread only
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<StreamWs> g_ws;  // a handful of entries: searched linearly

// The buffer of (current device, st) with at least `need` bytes; g_ws_mutex held by the caller.
int stream_workspace(hipStream_t st, size_t need, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  const std::thread::id tid = st == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
  StreamWs* w = nullptr;
  for (auto& c : g_ws)
    if (c.dev == dev && c.st == st && c.thread == tid) w = &c;
  if (!w) {
    try {
      g_ws.push_back(StreamWs{dev, st, tid, nullptr, 0});
    } catch (...) {
      return fail(HQQ_ERR_WORKSPACE, "no host memory for the workspace table");
    }
    w = &g_ws.back();
  }
  if (w->bytes < need) {
    if (w->ptr) {
      e = hipStreamSynchronize(st);  // the stream's earlier calls may still use the old buffer
      if (e != hipSuccess) return device_fail(e, "hipStreamSynchronize");
      e = hipFree(w->ptr);
      w->ptr = nullptr;
      w->bytes = 0;
      if (e != hipSuccess) return device_fail(e, "hipFree");
    }
    const size_t bytes = (need + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);  // whole MiB
    e = hipMalloc(&w->ptr, bytes);
    if (e != hipSuccess) {
      w->ptr = nullptr;
      return device_fail(e, "hipMalloc of the batched product's workspace");
    }
    w->bytes = bytes;
  }
  *out = w->ptr;
  return HQQ_OK;
}

}  // namespace

extern "C" {

int hqq_quantize_noalloc(const void* W_fp16, int64_t rows, int64_t cols, int nbits, int group_size, int axis,
                         int iters, double p, double beta0, double kappa, void* packed, void* delta, void* zero,
                         int meta_dtype, int32_t* stop_iter_dev, double* mae_trace_dev, void* stream) {
  g_last_error[0] = 0;
  // everything that can be checked without the device first: the shape, then the scratch need
  int st = check_shape(rows, cols, nbits, group_size, axis);
  if (st != HQQ_OK) return st;
  if (iters < 0 || iters > HQQ_MAX_ITERS) return fail(HQQ_ERR_INVALID_ARGUMENT, "iters must be in [0, %d]", HQQ_MAX_ITERS);
  QuantLayout q;
  if (!quant_layout(rows, cols, nbits, group_size, axis, iters, &q))
    return fail(HQQ_ERR_UNSUPPORTED, "configuration needs more LDS than one block may use");
  if (q.total > (size_t)HQQ_NOALLOC_SCRATCH_BYTES)
    return fail(HQQ_ERR_WORKSPACE, "this tensor needs %zu bytes of scratch, beyond the %zu of the allocation-free entry point",
                q.total, (size_t)HQQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != HQQ_OK) return st;
  const hqq_quant_args x = {W_fp16, rows, cols, nbits, group_size, axis, iters, p, beta0, kappa, packed, delta,
                            zero, meta_dtype, ws, (size_t)HQQ_NOALLOC_SCRATCH_BYTES, stop_iter_dev, mae_trace_dev,
                            stream, HQQ_STOP_BEST, HQQ_TINY_RANGE, 0};
  return quantize_impl(x);
}

int hqq_quantize_ex(const hqq_quant_args* args) {
  g_last_error[0] = 0;
  if (!args) return fail(HQQ_ERR_INVALID_ARGUMENT, "null args");
  const int r = args->stop_rule;
  if (r < 0 || r > 6 || (r & 3) == 3) return fail(HQQ_ERR_INVALID_ARGUMENT, "stop_rule must be 0, 1 or 2, optionally | 4");
  if (!(args->tiny_range >= 0.0) || !isfinite(args->tiny_range))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "tiny_range must be finite and >= 0");
  if (args->debug_flags & ~(HQQ_DEBUG_NO_FROZEN_SKIP | HQQ_DEBUG_SLOW_SHRINK | HQQ_DEBUG_SYNC))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "unknown debug flags");
  return quantize_impl(*args);
}

size_t hqq_quantize_v2_workspace_bytes(int64_t rows, int64_t cols, int nbits) {
  if (nbits != 3 || rows <= 0 || cols <= 0) return 0;
  return ((size_t)rows * (size_t)cols + 255) & ~size_t(255);  // one byte per code before packing
}

int hqq_quantize_v2(const hqq_quant_v2_args* args) {
  g_last_error[0] = 0;
  if (!args) return fail(HQQ_ERR_INVALID_ARGUMENT, "null args");
  const hqq_quant_v2_args& x = *args;
  int st = check_shape(x.rows, x.cols, x.nbits, x.group_size, x.axis);
  if (st != HQQ_OK) return st;
  if (x.iters < 0 || x.iters > HQQ_MAX_ITERS) return fail(HQQ_ERR_INVALID_ARGUMENT, "iters must be in [0, %d]", HQQ_MAX_ITERS);
  if (!(x.p > 0.0 && x.p <= 1.0)) return fail(HQQ_ERR_INVALID_ARGUMENT, "p must be in (0, 1]");
  if (!(x.beta0 > 0.0) || !isfinite(x.beta0)) return fail(HQQ_ERR_INVALID_ARGUMENT, "beta0 must be positive");
  if (!(x.kappa > 0.0) || !isfinite(x.kappa)) return fail(HQQ_ERR_INVALID_ARGUMENT, "kappa must be positive");
  if (!(x.tiny_range >= 0.0) || !isfinite(x.tiny_range))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "tiny_range must be finite and >= 0");
  if (x.n_candidates < 1 || x.n_candidates > HQQ_V2_MAX_CANDIDATES || !x.scale_grid)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "n_candidates must be in [1, %d] with a scale_grid", HQQ_V2_MAX_CANDIDATES);
  for (int c = 0; c < x.n_candidates; ++c)
    if (!(x.scale_grid[c] > 0.0) || !isfinite(x.scale_grid[c]))
      return fail(HQQ_ERR_INVALID_ARGUMENT, "scale_grid values must be finite and positive");
  if (x.meta_dtype != HQQ_META_F16 && x.meta_dtype != HQQ_META_F32 && x.meta_dtype != HQQ_META_F64)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "meta_dtype must be HQQ_META_F16, _F32 or _F64");
  if (!x.W_fp16 || !x.packed || !x.delta || !x.zero) return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(x.W_fp16) || !aligned16(x.packed) || !aligned16(x.delta) || !aligned16(x.zero))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const size_t wsb = hqq_quantize_v2_workspace_bytes(x.rows, x.cols, x.nbits);
  if (wsb && (!x.workspace || x.workspace_bytes < wsb))
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes needed", wsb);
  if (wsb && !aligned16(x.workspace)) return fail(HQQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  const int64_t G = x.rows * x.cols / x.group_size;  // >= 1: rows, cols > 0 and g divides cols

  hqq::SolveArgs a;
  memset(&a, 0, sizeof(a));
  a.W = reinterpret_cast<const __half*>(x.W_fp16);
  a.packed = reinterpret_cast<uint8_t*>(x.packed);
  a.delta = x.delta;
  a.zero = x.zero;
  a.codes_ws = x.nbits == 3 ? reinterpret_cast<uint8_t*>(x.workspace) : nullptr;
  a.G = G;
  a.nblocks = hqq::quant_v2_blocks(G, x.group_size);
  a.iters = x.iters;
  a.meta_dtype = x.meta_dtype;
  a.qmax = (double)((1 << x.nbits) - 1);
  a.tiny = x.tiny_range;
  a.pm1 = x.p - 1.0;
  fill_schedule(a, x.iters, x.p, x.beta0, x.kappa);
  hqq::ScaleGrid sg;
  memset(&sg, 0, sizeof(sg));
  for (int c = 0; c < x.n_candidates; ++c) sg.c[c] = x.scale_grid[c];
  sg.n = x.n_candidates;
  sg.choice = x.choice_dev;
  hipError_t e =
      hqq::launch_quantize_v2(a, sg, x.nbits, x.group_size, x.axis, reinterpret_cast<hipStream_t>(x.stream));
  if (e != hipSuccess) return device_fail(e, "hqq_quantize_v2 launch");
  return HQQ_OK;
}

int hqq_dequantize(const void* packed, const void* delta, const void* zero, int meta_dtype, int64_t rows,
                   int64_t cols, int nbits, int group_size, int axis, void* W_out_fp16, void* stream) {
  g_last_error[0] = 0;
  int st = check_shape(rows, cols, nbits, group_size, axis);
  if (st != HQQ_OK) return st;
  if (meta_dtype != HQQ_META_F16 && meta_dtype != HQQ_META_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "meta_dtype must be HQQ_META_F16 or HQQ_META_F32");
  if (!packed || !delta || !zero || !W_out_fp16) return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta) || !aligned16(zero) || !aligned16(W_out_fp16))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  hipError_t e = hqq::launch_dequant(reinterpret_cast<const uint8_t*>(packed), delta, zero, meta_dtype, rows, cols,
                                     nbits, group_size, axis, reinterpret_cast<__half*>(W_out_fp16),
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "hqq_dequantize launch");
  return HQQ_OK;
}

int hqq_gemv_w4a16(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                   int group_size, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* stream) {
  g_last_error[0] = 0;
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || batch > (int64_t(1) << 24))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (group_size <= 0 || K % group_size != 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide K");
  if (group_size != 64 && group_size != 128) return fail(HQQ_ERR_UNSUPPORTED, "group_size must be 64 or 128");
  if (N % 16 != 0 || K % 128 != 0) return fail(HQQ_ERR_UNSUPPORTED, "N must be a multiple of 16 and K of 128");
  if (y_dtype != HQQ_OUT_F16 && y_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "y_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !x_fp16 || !y) return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(x_fp16) || !aligned16(y))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* pk = reinterpret_cast<const uint8_t*>(packed);
  const __half* dl = reinterpret_cast<const __half*>(delta_fp16);
  const __half* zr = reinterpret_cast<const __half*>(zero_fp16);
  const __half* xx = reinterpret_cast<const __half*>(x_fp16);
  hipError_t e;
  // Batch 3-16 on up to 2^24 weights (batch 9-16 on up to 2^26) runs the kernel that dequantises
  // its tile in registers into the MFMA (measured faster there: 4096 x 4096 batch 8 7.9 against
  // 11.1 us, 11008 x 4096 batch 9 17.5 against 30.3 us through the split GEMM); larger weights
  // keep the segment-pipelined MFMA GEMV (batch 3-8) or the split GEMM.
  const bool dq = batch >= 3 && batch <= 16 && N * K <= (batch <= 8 ? (int64_t(1) << 24) : (int64_t(1) << 26)) &&
                  hqq::gemv_dq_supported(N, K, 4, group_size, batch);
  if (dq) {
    e = hqq::launch_gemv_dq(pk, dl, zr, N, K, 4, group_size, xx, batch, y, y_dtype, st);
  } else if (batch <= 8) {
    if (hqq::gemv_lds_bytes(K, group_size, batch) > 160 * 1024) return fail(HQQ_ERR_UNSUPPORTED, "LDS too large");  // 160 KB per workgroup on gfx950
    e = hqq::launch_gemv(pk, dl, zr, N, K, group_size, xx, batch, y, y_dtype, st);
  } else if (hqq::gemm_splits(N, K, batch) != 0) {  // the split GEMM on the stream's workspace
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    void* ws = nullptr;
    const int s = stream_workspace(st, hqq::gemm_workspace_bytes(N, K, batch), &ws);
    if (s != HQQ_OK) return s;
    e = hqq::launch_gemm_split(pk, dl, zr, N, K, group_size, xx, batch, y, y_dtype, ws, st);
  } else {
    e = hqq::launch_gemm(pk, dl, zr, N, K, group_size, xx, batch, y, y_dtype, st);
  }
  if (e != hipSuccess) return device_fail(e, "hqq_gemv_w4a16 launch");
  return HQQ_OK;
}

int hqq_release_workspaces(void) {
  g_last_error[0] = 0;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  int status = HQQ_OK;
  for (auto& c : g_ws) {
    if (!c.ptr) continue;
    e = hipSetDevice(c.dev);
    if (e == hipSuccess) e = hipFree(c.ptr);  // waits for the device's work
    if (e != hipSuccess && status == HQQ_OK) status = device_fail(e, "hipFree of a workspace");
  }
  g_ws.clear();
  e = hipSetDevice(cur);
  if (e != hipSuccess && status == HQQ_OK) status = device_fail(e, "hipSetDevice");
  return status;
}

size_t hqq_gemm_workspace_bytes(int64_t N, int64_t K, int64_t batch) {
  if (N <= 0 || K <= 0 || batch <= 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31) ||
      batch > (int64_t(1) << 24))
    return 0;
  return hqq::gemm_workspace_bytes(N, K, batch);
}

int hqq_gemm_w4a16(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                   int group_size, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || batch > (int64_t(1) << 24))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (group_size <= 0 || K % group_size != 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide K");
  if (group_size != 64 && group_size != 128) return fail(HQQ_ERR_UNSUPPORTED, "group_size must be 64 or 128");
  if (hqq::gemm_splits(N, K, batch) == 0)
    return fail(HQQ_ERR_UNSUPPORTED, "N must be a multiple of 128 and K of 256");
  if (y_dtype != HQQ_OUT_F16 && y_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "y_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !x_fp16 || !y || !workspace)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(x_fp16) || !aligned16(y) ||
      !aligned16(workspace))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const size_t need = hqq::gemm_workspace_bytes(N, K, batch);
  if (workspace_bytes < need)
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const hipError_t e = hqq::launch_gemm_split(
      reinterpret_cast<const uint8_t*>(packed), reinterpret_cast<const __half*>(delta_fp16),
      reinterpret_cast<const __half*>(zero_fp16), N, K, group_size, reinterpret_cast<const __half*>(x_fp16), batch, y,
      y_dtype, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "hqq_gemm_w4a16 launch");
  return HQQ_OK;
}

int hqq_gemm(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
             int group_size, int axis, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || batch > (int64_t(1) << 24))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (nbits != 2 && nbits != 3 && nbits != 4) return fail(HQQ_ERR_INVALID_ARGUMENT, "nbits must be 2, 3 or 4");
  if (axis != 0 && axis != 1) return fail(HQQ_ERR_INVALID_ARGUMENT, "axis must be 0 or 1");
  if (group_size <= 0 || (axis == 1 ? K : N) % group_size != 0)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide the grouped dimension");
  if (axis == 0 && nbits != 4) return fail(HQQ_ERR_UNSUPPORTED, "the batched product takes axis-0 groups at 4 bits");
  if (nbits == 4 && axis == 1 ? (group_size != 64 && group_size != 128) : !pow2_group(group_size))
    return fail(HQQ_ERR_UNSUPPORTED,
                "group_size 64 or 128 for 4-bit axis-1 codes, a power of two 16..256 for 2/3-bit or axis-0 codes");
  if (hqq::gemm_splits(N, K, batch) == 0)
    return fail(HQQ_ERR_UNSUPPORTED, "N must be a multiple of 128 and K of 256");
  if (y_dtype != HQQ_OUT_F16 && y_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "y_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !x_fp16 || !y || !workspace)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(x_fp16) || !aligned16(y) ||
      !aligned16(workspace))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const size_t need = hqq::gemm_workspace_bytes(N, K, batch);
  if (workspace_bytes < need)
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const hipError_t e = hqq::launch_gemm_fmt(
      reinterpret_cast<const uint8_t*>(packed), reinterpret_cast<const __half*>(delta_fp16),
      reinterpret_cast<const __half*>(zero_fp16), N, K, nbits, group_size, axis,
      reinterpret_cast<const __half*>(x_fp16), batch, y, y_dtype, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "hqq_gemm launch");
  return HQQ_OK;
}

size_t hqq_gemm_dx_workspace_bytes(int64_t N, int64_t K, int64_t batch) {
  if (N <= 0 || K <= 0 || batch <= 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31) ||
      batch > (int64_t(1) << 24))
    return 0;
  return hqq::gemm_workspace_bytes(K, N, batch);
}

int hqq_gemm_w4a16_dx(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K,
                      int group_size, const void* dy_fp16, int64_t batch, void* dx, int dx_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || batch > (int64_t(1) << 24))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (group_size <= 0 || K % group_size != 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide K");
  if (group_size != 64 && group_size != 128) return fail(HQQ_ERR_UNSUPPORTED, "group_size must be 64 or 128");
  if (hqq::gemm_splits(K, N, batch) == 0)
    return fail(HQQ_ERR_UNSUPPORTED, "K must be a multiple of 128 and N of 256");
  if (dx_dtype != HQQ_OUT_F16 && dx_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "dx_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !dy_fp16 || !dx || !workspace)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(dy_fp16) || !aligned16(dx) ||
      !aligned16(workspace))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const size_t need = hqq::gemm_workspace_bytes(K, N, batch);
  if (workspace_bytes < need)
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const hipError_t e = hqq::launch_gemm_dx(
      reinterpret_cast<const uint8_t*>(packed), reinterpret_cast<const __half*>(delta_fp16),
      reinterpret_cast<const __half*>(zero_fp16), N, K, 4, group_size, 1, reinterpret_cast<const __half*>(dy_fp16),
      batch, dx, dx_dtype, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "hqq_gemm_w4a16_dx launch");
  return HQQ_OK;
}

int hqq_gemm_dx(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
                int group_size, int axis, const void* dy_fp16, int64_t batch, void* dx, int dx_dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || batch > (int64_t(1) << 24))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (nbits != 2 && nbits != 3 && nbits != 4) return fail(HQQ_ERR_INVALID_ARGUMENT, "nbits must be 2, 3 or 4");
  if (axis != 0 && axis != 1) return fail(HQQ_ERR_INVALID_ARGUMENT, "axis must be 0 or 1");
  if (group_size <= 0 || (axis == 1 ? K : N) % group_size != 0)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide the grouped dimension");
  if (axis == 0 && nbits != 4) return fail(HQQ_ERR_UNSUPPORTED, "the input gradient takes axis-0 groups at 4 bits");
  if (nbits == 4 && axis == 1 ? (group_size != 64 && group_size != 128) : !pow2_group(group_size))
    return fail(HQQ_ERR_UNSUPPORTED,
                "group_size 64 or 128 for 4-bit axis-1 codes, a power of two 16..256 for 2/3-bit or axis-0 codes");
  if (hqq::gemm_splits(K, N, batch) == 0)
    return fail(HQQ_ERR_UNSUPPORTED, "K must be a multiple of 128 and N of 256");
  if (dx_dtype != HQQ_OUT_F16 && dx_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "dx_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !dy_fp16 || !dx || !workspace)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(dy_fp16) || !aligned16(dx) ||
      !aligned16(workspace))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const size_t need = hqq::gemm_workspace_bytes(K, N, batch);
  if (workspace_bytes < need)
    return fail(HQQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const hipError_t e = hqq::launch_gemm_dx(
      reinterpret_cast<const uint8_t*>(packed), reinterpret_cast<const __half*>(delta_fp16),
      reinterpret_cast<const __half*>(zero_fp16), N, K, nbits, group_size, axis,
      reinterpret_cast<const __half*>(dy_fp16), batch, dx, dx_dtype, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "hqq_gemm_dx launch");
  return HQQ_OK;
}

int hqq_gemv(const void* packed, const void* delta_fp16, const void* zero_fp16, int64_t N, int64_t K, int nbits,
             int group_size, int axis, const void* x_fp16, int64_t batch, void* y, int y_dtype, void* stream) {
  g_last_error[0] = 0;
  if (nbits == 4 && axis == 1)
    return hqq_gemv_w4a16(packed, delta_fp16, zero_fp16, N, K, group_size, x_fp16, batch, y, y_dtype, stream);
  if (N <= 0 || K <= 0 || batch <= 0) return fail(HQQ_ERR_INVALID_ARGUMENT, "N, K and batch must be positive");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return fail(HQQ_ERR_INVALID_ARGUMENT, "shape too large");
  if (nbits != 2 && nbits != 3 && nbits != 4) return fail(HQQ_ERR_INVALID_ARGUMENT, "nbits must be 2, 3 or 4");
  if (axis != 0 && axis != 1) return fail(HQQ_ERR_INVALID_ARGUMENT, "axis must be 0 or 1");
  if (group_size <= 0 || (axis == 1 ? K : N) % group_size != 0)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "group_size must divide %s", axis == 1 ? "K" : "N");
  if (y_dtype != HQQ_OUT_F16 && y_dtype != HQQ_OUT_F32)
    return fail(HQQ_ERR_INVALID_ARGUMENT, "y_dtype must be HQQ_OUT_F16 or HQQ_OUT_F32");
  if (!packed || !delta_fp16 || !zero_fp16 || !x_fp16 || !y) return fail(HQQ_ERR_INVALID_ARGUMENT, "null buffer");
  if (!aligned16(packed) || !aligned16(delta_fp16) || !aligned16(zero_fp16) || !aligned16(x_fp16) || !aligned16(y))
    return fail(HQQ_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  if (batch > (nbits == 4 ? 8 : 16))
    return fail(HQQ_ERR_UNSUPPORTED, "batch must be at most 8 for axis-0 4-bit codes and 16 for 3/2-bit codes");
  if (batch <= 2 && K > 16384) return fail(HQQ_ERR_UNSUPPORTED, "K must be at most 16384 for this format");
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* pk = reinterpret_cast<const uint8_t*>(packed);
  const __half* dl = reinterpret_cast<const __half*>(delta_fp16);
  const __half* zr = reinterpret_cast<const __half*>(zero_fp16);
  const __half* xx = reinterpret_cast<const __half*>(x_fp16);
  hipError_t e;
  if (batch > 2 && axis == 1) {  // 3/2-bit codes, batch 3-16: the tile dequantised in registers into the MFMA
    if (nbits == 2 && group_size != 16)
      return fail(HQQ_ERR_UNSUPPORTED, "no fused product for nbits=2 group_size=%d", group_size);
    if (!hqq::gemv_dq_supported(N, K, nbits, group_size, batch))
      return fail(HQQ_ERR_UNSUPPORTED, "batch 3-16: K must be a multiple of 128 and at most %s, group_size 16..256",
                  nbits == 3 ? "12288 (24576 with at most 8160 rows)" : "16384 (32768 with at most 8160 rows)");
    e = hqq::launch_gemv_dq(pk, dl, zr, N, K, nbits, group_size, xx, batch, y, y_dtype, st);
  } else if (nbits == 4 && axis == 0) {
    if (!pow2_group(group_size)) return fail(HQQ_ERR_UNSUPPORTED, "group_size must be 16, 32, 64, 128 or 256");
    if (K % 32 != 0) return fail(HQQ_ERR_UNSUPPORTED, "K must be a multiple of 32");
    if (batch > 2 && K % 128 != 0) return fail(HQQ_ERR_UNSUPPORTED, "batch 3-8: K must be a multiple of 128");
    if (hqq::gemv_ax0_lds_bytes(K, batch) > 160 * 1024) return fail(HQQ_ERR_UNSUPPORTED, "LDS too large");
    e = hqq::launch_gemv_ax0(pk, dl, zr, N, K, group_size, xx, batch, y, y_dtype, st);
  } else if (nbits == 3 && axis == 1) {
    if (!hqq::gemv_3b_supported(K, group_size))
      return fail(HQQ_ERR_UNSUPPORTED, "3-bit: pow2 group_size 16..256 and K of at most 8192");
    if (N % 4 != 0) return fail(HQQ_ERR_UNSUPPORTED, "3-bit: N must be a multiple of 4");
    if (hqq::gemv_3b_lds_bytes(N, K, group_size, batch) > 160 * 1024) return fail(HQQ_ERR_UNSUPPORTED, "LDS too large");
    e = hqq::launch_gemv_3b(pk, dl, zr, N, K, group_size, xx, batch, y, y_dtype, st);
  } else if (nbits == 2 && axis == 1 && group_size == 16) {
    if (N % 16 != 0 || K % 64 != 0) return fail(HQQ_ERR_UNSUPPORTED, "N must be a multiple of 16 and K of 64");
    e = hqq::launch_gemv_2b(pk, dl, zr, N, K, xx, batch, y, y_dtype, st);
  } else {
    return fail(HQQ_ERR_UNSUPPORTED, "no fused product for nbits=%d group_size=%d axis=%d", nbits, group_size, axis);
  }
  if (e != hipSuccess) return device_fail(e, "hqq_gemv launch");
  return HQQ_OK;
}

const char* hqq_status_string(int status) {
  switch (status) {
    case HQQ_OK: return "HQQ_OK";
    case HQQ_ERR_INVALID_ARGUMENT: return "HQQ_ERR_INVALID_ARGUMENT";
    case HQQ_ERR_UNSUPPORTED: return "HQQ_ERR_UNSUPPORTED";
    case HQQ_ERR_WORKSPACE: return "HQQ_ERR_WORKSPACE";
    case HQQ_ERR_DEVICE: return "HQQ_ERR_DEVICE";
    default: return "HQQ_ERR_UNKNOWN";
  }
}

const char* hqq_last_error(void) { return g_last_error; }

}  // extern "C"
