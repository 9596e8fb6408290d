// Standalone dequantisation (page "HQQ 算法解读", sections "量化公式" and "从压缩文件到一次前向"):
// W_hat = (q - zero) * delta per group, written as fp16.
//
// HBM-streaming: each thread turns one 32-bit word of packed codes (8 4-bit, 16 2-bit or
// 10 3-bit codes) into fp16 outputs with vector stores.  The product (q - z) * delta is
// formed in fp32 (q - z is exact for |z| >= 2^-10 or z = 0 with fp16 metadata), its rounding
// error is recovered with one fma and folded in as a sticky bit (round to odd), so the single
// fp32 -> fp16 conversion rounds the exact product to nearest even.

#include "hqq_internal.h"

namespace hqq {
namespace {

__device__ __forceinline__ unsigned short dq(float q, float z, float d) {
  const float a = q - z;
  const float p = a * d;
  const float err = fmaf(a, d, -p);
  unsigned u = __float_as_uint(p);
  if (err != 0.0f) {
    if ((err < 0.0f) == (p > 0.0f)) u -= 1u;  // p was rounded away from zero: step back
    u |= 1u;
  }
  return __half_as_ushort(__float2half_rn(__uint_as_float(u)));
}

template <int META>
__device__ __forceinline__ float meta_at(const void* p, int64_t j) {
  if constexpr (META == HQQ_META_F16)
    return __half2float(reinterpret_cast<const __half*>(p)[j]);
  else
    return reinterpret_cast<const float*>(p)[j];
}

// 4-bit or 2-bit: one 32-bit word per thread (8 or 16 codes, flat index base = 8w or 16w).
template <int NBITS, int AXIS, int META>
__global__ void __launch_bounds__(256) k_dequant_word(const uint32_t* packed, const void* delta, const void* zero,
                                                      int64_t nwords, int64_t M, int gshift, __half* out) {
  constexpr int CPW = 32 / NBITS;  // codes per word
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nwords) return;
  const uint32_t word = packed[w];
  const int64_t base = w * CPW;
  unsigned short h[CPW];
  if constexpr (AXIS == 1) {
    // CPW <= group size: the whole word is one group
    const int64_t j = base >> gshift;
    const float z = meta_at<META>(zero, j), d = meta_at<META>(delta, j);
#pragma unroll
    for (int t = 0; t < CPW; ++t) h[t] = dq((float)((word >> (NBITS * t)) & ((1u << NBITS) - 1)), z, d);
  } else {
    // consecutive codes belong to consecutive groups (group of flat index i is i mod M)
    const int64_t j0 = base % M;
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
      int64_t j = j0 + t;
      if (j >= M) j -= M;
      h[t] = dq((float)((word >> (NBITS * t)) & ((1u << NBITS) - 1)), meta_at<META>(zero, j),
                meta_at<META>(delta, j));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(out + base);
#pragma unroll
  for (int v = 0; v < CPW / 8; ++v)
    dst[v] = make_uint4(h[8 * v] | ((unsigned)h[8 * v + 1] << 16), h[8 * v + 2] | ((unsigned)h[8 * v + 3] << 16),
                        h[8 * v + 4] | ((unsigned)h[8 * v + 5] << 16), h[8 * v + 6] | ((unsigned)h[8 * v + 7] << 16));
}

// 3-bit: one word = 10 codes per thread (flat index base = 10w), the last word partial.
template <int AXIS, int META>
__global__ void __launch_bounds__(256) k_dequant3(const uint32_t* packed, const void* delta, const void* zero,
                                                  int64_t N, int64_t nwords, int64_t M, int gshift, __half* out) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nwords) return;
  const uint32_t word = packed[w];
  const int64_t base = w * 10;
  unsigned short h[10];
  const int64_t j0 = (AXIS == 1) ? 0 : base % M;
#pragma unroll
  for (int t = 0; t < 10; ++t) {
    const int64_t i = base + t;
    int64_t j;
    if (AXIS == 1) {
      j = i >> gshift;
    } else {
      j = j0 + t;
      if (j >= M) j -= M;
    }
    const int64_t jj = i < N ? j : 0;
    h[t] = dq((float)((word >> (3 * t)) & 7u), meta_at<META>(zero, jj), meta_at<META>(delta, jj));
  }
  if (base + 10 <= N) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + base);  // 20-byte rows: 4-byte aligned
#pragma unroll
    for (int v = 0; v < 5; ++v) dst[v] = h[2 * v] | ((unsigned)h[2 * v + 1] << 16);
  } else {
    unsigned short* dst = reinterpret_cast<unsigned short*>(out + base);
    for (int t = 0; base + t < N; ++t) dst[t] = h[t];
  }
}

template <int NBITS, int AXIS>
hipError_t dispatch_meta(const uint8_t* packed, const void* delta, const void* zero, int meta, int64_t N,
                         int64_t M, int gshift, __half* out, hipStream_t st) {
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  if constexpr (NBITS == 3) {
    const int64_t nwords = (N + 9) / 10;
    const dim3 grid((unsigned)((nwords + 255) / 256));
    if (meta == HQQ_META_F16)
      hipLaunchKernelGGL((k_dequant3<AXIS, HQQ_META_F16>), grid, dim3(256), 0, st, pk, delta, zero, N, nwords, M,
                         gshift, out);
    else
      hipLaunchKernelGGL((k_dequant3<AXIS, HQQ_META_F32>), grid, dim3(256), 0, st, pk, delta, zero, N, nwords, M,
                         gshift, out);
  } else {
    const int64_t nwords = N / (32 / NBITS);
    const dim3 grid((unsigned)((nwords + 255) / 256));
    if (meta == HQQ_META_F16)
      hipLaunchKernelGGL((k_dequant_word<NBITS, AXIS, HQQ_META_F16>), grid, dim3(256), 0, st, pk, delta, zero,
                         nwords, M, gshift, out);
    else
      hipLaunchKernelGGL((k_dequant_word<NBITS, AXIS, HQQ_META_F32>), grid, dim3(256), 0, st, pk, delta, zero,
                         nwords, M, gshift, out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t* packed, const void* delta, const void* zero, int meta, int64_t rows,
                          int64_t cols, int nbits, int g, int axis, __half* out, hipStream_t st) {
  const int64_t N = rows * cols;
  const int64_t M = N / g;
  int gshift = 0;
  while ((1 << gshift) < g) ++gshift;
  if (nbits == 4)
    return axis == 1 ? dispatch_meta<4, 1>(packed, delta, zero, meta, N, M, gshift, out, st)
                     : dispatch_meta<4, 0>(packed, delta, zero, meta, N, M, gshift, out, st);
  if (nbits == 2)
    return axis == 1 ? dispatch_meta<2, 1>(packed, delta, zero, meta, N, M, gshift, out, st)
                     : dispatch_meta<2, 0>(packed, delta, zero, meta, N, M, gshift, out, st);
  return axis == 1 ? dispatch_meta<3, 1>(packed, delta, zero, meta, N, M, gshift, out, st)
                   : dispatch_meta<3, 0>(packed, delta, zero, meta, N, M, gshift, out, st);
}

}  // namespace hqq
