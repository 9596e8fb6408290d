// Standalone dequantisation (page "HQQ 算法解读", sections "量化公式" and "从压缩文件到一次前向"):
// W_hat = (q - zero) * delta per group, written as fp16, the exact product rounded once to
// nearest even.
//
// fp16 metadata (the stored format): a code c masked into an fp16 subnormal field at bit
// position m reads as c 2^(m-24); with ds = delta 2^(24-m) and zd = zero delta (exact in fp32:
// 11 x 11 significant bits), the mixed-precision FMA with an fp16 result,
// fma(c 2^(m-24), ds, -zd), forms (c - zero) delta exactly and rounds it once (this rounding,
// subnormal results included, was checked against the exact product on gfx950).  That is two
// or three VALU operations per code, so these kernels stay HBM-bound.  A zero result is +0
// where delta <= 0 would give -0 (delta = 1/s > 0 for every quantizer output).
// Output is written with non-temporal stores, each instruction covering 1 KB of consecutive
// bytes (2-bit and 3-bit results are restaged through LDS to get there): the streamed result
// then leaves no dirty lines in L2 for the end of the kernel to write back, and no store
// instruction leaves a partial line.
//
// fp32 metadata, and the fp16 layouts without a fast form (3-bit axis 0, 2-bit axis 0 with
// (rows/g) cols not a multiple of 16): the product is formed in fp32 (q - z is exact for
// |z| >= 2^-10 or z = 0), its rounding error recovered with one fma and folded in as a
// sticky bit (round to odd), so the single fp32 -> fp16 conversion rounds the exact product.

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

// ------------------------------------------------------------------ fp16 metadata, mixed FMA
// Operand forms (VOP3P mixed precision): op_sel picks the high fp16 half of a source,
// op_sel_hi marks a source as fp16.
#define HQQ_MIXLO(NAME, SEL)                                                                        \
  __device__ __forceinline__ unsigned NAME(unsigned t, float ds, float zd) {                        \
    unsigned r;                                                                                     \
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[" #SEL ",0,0] op_sel_hi:[1,0,0]"                   \
        : "=v"(r) : "v"(t), "v"(ds), "v"(zd));                                                      \
    return r;                                                                                       \
  }
#define HQQ_MIXHI(NAME, SEL)                                                                        \
  __device__ __forceinline__ void NAME(unsigned& r, unsigned t, float ds, float zd) {               \
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[" #SEL ",0,0] op_sel_hi:[1,0,0]"                   \
        : "+v"(r) : "v"(t), "v"(ds), "v"(zd));                                                      \
  }
typedef unsigned u32x4n __attribute__((ext_vector_type(4)));

// 16-byte non-temporal store
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
  const u32x4n w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4n*>(p));
}

HQQ_MIXLO(mixlo0, 0)
HQQ_MIXLO(mixlo1, 1)
HQQ_MIXHI(mixhi0, 0)
HQQ_MIXHI(mixhi1, 1)
#undef HQQ_MIXLO
#undef HQQ_MIXHI

// out = fp16(c_lo-or-hi * ds - zd) into the low (LO = true) or high half of r
template <int SEL, bool LO>
__device__ __forceinline__ void put(unsigned& r, unsigned t, float ds, float zd) {
  if constexpr (LO) r = SEL ? mixlo1(t, ds, zd) : mixlo0(t, ds, zd);
  else if constexpr (SEL) mixhi1(r, t, ds, zd);
  else mixhi0(r, t, ds, zd);
}

// x.half[S] * y.half[S], both fp16, exact in fp32
template <int S>
__device__ __forceinline__ float hmul(unsigned x, unsigned y) {
  float r;
  if constexpr (S == 0)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(x), "v"(y));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

// x.half[SX] (fp16) * s (fp32, a power of two): exact
template <int SX>
__device__ __forceinline__ float hscale(unsigned x, float s) {
  float r;
  if constexpr (SX == 0)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(s));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(s));
  return r;
}

__device__ __forceinline__ float p2(int e) { return __uint_as_float((unsigned)(127 + e) << 23); }

// 8 4-bit codes of word w, one (ds24, ds20, zd) for all: 4 dwords of fp16 in code order.
// t0 = (c0, c4), t1 = 16 (c1, c5), t2 = (c2, c6), t3 = 16 (c3, c7) in the (low, high) halves.
__device__ __forceinline__ uint4 dq4_word(unsigned w, float ds24, float ds20, float zd) {
  const unsigned t0 = w & 0x000F000Fu, t1 = w & 0x00F000F0u, u = w >> 8;
  const unsigned t2 = u & 0x000F000Fu, t3 = u & 0x00F000F0u;
  uint4 o;
  put<0, true>(o.x, t0, ds24, zd);
  put<0, false>(o.x, t1, ds20, zd);
  put<0, true>(o.y, t2, ds24, zd);
  put<0, false>(o.y, t3, ds20, zd);
  put<1, true>(o.z, t0, ds24, zd);
  put<1, false>(o.z, t1, ds20, zd);
  put<1, true>(o.w, t2, ds24, zd);
  put<1, false>(o.w, t3, ds20, zd);
  return o;
}

// 16 2-bit codes of word w: pair masks give (c_k, c_{k+8}) at bit 2k mod 8 (scales 2^24..2^18).
__device__ __forceinline__ void dq2_word(unsigned w, const float (&ds)[4], float zd, uint4& o0, uint4& o1) {
  const unsigned u = w >> 8;
  const unsigned t[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u,
                         u & 0x00030003u, u & 0x000C000Cu, u & 0x00300030u, u & 0x00C000C0u};
  unsigned r[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // t[m] holds its codes at bit 2 (m mod 4) of the half: scale ds[m mod 4]
    put<0, true>(r[k], t[2 * k], ds[(2 * k) % 4], zd);
    put<0, false>(r[k], t[2 * k + 1], ds[(2 * k + 1) % 4], zd);
    put<1, true>(r[4 + k], t[2 * k], ds[(2 * k) % 4], zd);
    put<1, false>(r[4 + k], t[2 * k + 1], ds[(2 * k + 1) % 4], zd);
  }
  o0 = make_uint4(r[0], r[1], r[2], r[3]);
  o1 = make_uint4(r[4], r[5], r[6], r[7]);
}

// 4-bit / 2-bit, axis 1: each wave takes U runs of 64 consecutive words (one word per lane,
// each inside one group).  4-bit: a lane's 16 output bytes are consecutive with its
// neighbours'.  2-bit: a lane's 32 bytes go through LDS so that each store instruction writes
// one half of the wave's 2 KB.
template <int NBITS, int U>
__global__ void __launch_bounds__(256) k_dqh_ax1(const uint32_t* __restrict__ packed,
                                                 const unsigned short* __restrict__ delta,
                                                 const unsigned short* __restrict__ zero, int64_t nwords,
                                                 int wshift, __half* __restrict__ out) {
  constexpr int CPW = 32 / NBITS;
  __shared__ uint4 stage[NBITS == 2 ? 4 : 1][NBITS == 2 ? 128 : 1];
  const int lane = threadIdx.x & 63, wi = threadIdx.x >> 6;
  const int64_t wb = (int64_t)blockIdx.x * (256 * U) + wi * 64 * U;  // first word of this wave
  unsigned wv[U], zv[U], dv[U];
#pragma unroll
  for (int v = 0; v < U; ++v) {
    const int64_t w = min(wb + 64 * v + lane, nwords - 1);
    wv[v] = packed[w];
    const int64_t j = w >> wshift;  // words per group = 2^wshift
    zv[v] = zero[j];
    dv[v] = delta[j];
  }
#pragma unroll
  for (int v = 0; v < U; ++v) {
    const int64_t w0 = wb + 64 * v;  // word of lane 0 in this run
    const float zd = hmul<0>(zv[v], dv[v]);
    uint4* dst = reinterpret_cast<uint4*>(out + w0 * CPW);
    if constexpr (NBITS == 4) {
      const uint4 o = dq4_word(wv[v], hscale<0>(dv[v], p2(24)), hscale<0>(dv[v], p2(20)), zd);
      if (w0 + lane < nwords) st_nt(dst + lane, o);
    } else {
      const float ds[4] = {hscale<0>(dv[v], p2(24)), hscale<0>(dv[v], p2(22)), hscale<0>(dv[v], p2(20)),
                           hscale<0>(dv[v], p2(18))};
      uint4 o0, o1;
      dq2_word(wv[v], ds, zd, o0, o1);
      stage[wi][2 * lane] = o0;
      stage[wi][2 * lane + 1] = o1;
      __builtin_amdgcn_wave_barrier();
      const uint4 lo = stage[wi][lane], hi = stage[wi][lane + 64];  // 16-byte pieces lane, lane + 64
      if (w0 + lane / 2 < nwords) st_nt(dst + lane, lo);
      if (w0 + 32 + lane / 2 < nwords) st_nt(dst + 64 + lane, hi);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// 4-bit / 2-bit, axis 0 (group of flat element i is i mod M): thread = one chunk of CPW
// consecutive groups (M % CPW == 0, so a word never wraps) and U of the g rows of the group.
template <int NBITS, int U>
__global__ void __launch_bounds__(256) k_dqh_ax0(const uint32_t* __restrict__ packed, const uint4* __restrict__ delta,
                                                 const uint4* __restrict__ zero, int64_t chunks, int g,
                                                 __half* __restrict__ out) {
  constexpr int CPW = 32 / NBITS;
  constexpr int V = CPW / 8;  // uint4 blocks of metadata per chunk
  __shared__ uint4 stage[NBITS == 2 ? 4 : 1][NBITS == 2 ? 128 : 1];
  const int lane = threadIdx.x & 63, wi = threadIdx.x >> 6;
  const int64_t c_lane0 = (int64_t)blockIdx.x * 256 + wi * 64;  // chunk of lane 0
  const int64_t c = min((int64_t)blockIdx.x * 256 + threadIdx.x, chunks - 1);
  const bool live = (int64_t)blockIdx.x * 256 + threadIdx.x < chunks;
  const int i0 = blockIdx.y * U;
  unsigned wv[U];
#pragma unroll
  for (int v = 0; v < U; ++v) wv[v] = packed[(int64_t)min(i0 + v, g - 1) * chunks + c];
  unsigned zq[4 * V], dq_[4 * V];
#pragma unroll
  for (int b = 0; b < V; ++b) {
    const uint4 z = zero[c * V + b], d = delta[c * V + b];
    zq[4 * b] = z.x, zq[4 * b + 1] = z.y, zq[4 * b + 2] = z.z, zq[4 * b + 3] = z.w;
    dq_[4 * b] = d.x, dq_[4 * b + 1] = d.y, dq_[4 * b + 2] = d.z, dq_[4 * b + 3] = d.w;
  }
  // per code k: zd_k and ds_k (its bit position's scale); code k sits in dword k/2, half k%2
  float zd[CPW], ds[CPW];
#pragma unroll
  for (int k = 0; k < CPW; k += 2) {
    zd[k] = hmul<0>(zq[k / 2], dq_[k / 2]);
    zd[k + 1] = hmul<1>(zq[k / 2], dq_[k / 2]);
  }
  if constexpr (NBITS == 4) {
    // code k: even k at bit 0 of its field (2^24), odd k at bit 4 (2^20)
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      ds[k] = hscale<0>(dq_[k / 2], p2(24));
      ds[k + 1] = hscale<1>(dq_[k / 2], p2(20));
    }
  } else {
    // code k at bit 2 (k mod 4) of its byte
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      ds[k] = hscale<0>(dq_[k / 2], p2(24 - 2 * (k % 4)));
      ds[k + 1] = hscale<1>(dq_[k / 2], p2(24 - 2 * ((k + 1) % 4)));
    }
  }
#pragma unroll
  for (int v = 0; v < U; ++v) {
    const unsigned w = wv[v];
    if constexpr (NBITS == 4) {
      uint4* dst = reinterpret_cast<uint4*>(out + ((int64_t)(i0 + v) * chunks + c) * CPW);
      const bool ok = live && i0 + v < g;
      const unsigned t0 = w & 0x000F000Fu, t1 = w & 0x00F000F0u, u = w >> 8;
      const unsigned t2 = u & 0x000F000Fu, t3 = u & 0x00F000F0u;
      uint4 o;
      put<0, true>(o.x, t0, ds[0], zd[0]);
      put<0, false>(o.x, t1, ds[1], zd[1]);
      put<0, true>(o.y, t2, ds[2], zd[2]);
      put<0, false>(o.y, t3, ds[3], zd[3]);
      put<1, true>(o.z, t0, ds[4], zd[4]);
      put<1, false>(o.z, t1, ds[5], zd[5]);
      put<1, true>(o.w, t2, ds[6], zd[6]);
      put<1, false>(o.w, t3, ds[7], zd[7]);
      if (ok) st_nt(dst, o);
    } else {
      const unsigned u = w >> 8;
      const unsigned t[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u,
                             u & 0x00030003u, u & 0x000C000Cu, u & 0x00300030u, u & 0x00C000C0u};
      unsigned r[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        put<0, true>(r[k], t[2 * k], ds[2 * k], zd[2 * k]);
        put<0, false>(r[k], t[2 * k + 1], ds[2 * k + 1], zd[2 * k + 1]);
        put<1, true>(r[4 + k], t[2 * k], ds[8 + 2 * k], zd[8 + 2 * k]);
        put<1, false>(r[4 + k], t[2 * k + 1], ds[8 + 2 * k + 1], zd[8 + 2 * k + 1]);
      }
      stage[wi][2 * lane] = make_uint4(r[0], r[1], r[2], r[3]);
      stage[wi][2 * lane + 1] = make_uint4(r[4], r[5], r[6], r[7]);
      __builtin_amdgcn_wave_barrier();
      const uint4 lo = stage[wi][lane], hi = stage[wi][lane + 64];
      uint4* row = reinterpret_cast<uint4*>(out + ((int64_t)(i0 + v) * chunks + c_lane0) * CPW);
      if (i0 + v < g) {
        if (c_lane0 + lane / 2 < chunks) st_nt(row + lane, lo);
        if (c_lane0 + 32 + lane / 2 < chunks) st_nt(row + 64 + lane, hi);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// 3-bit, axis 1: thread T takes words 4T..4T+3 (codes 40T..40T+39, 80 output bytes).  The
// 40 codes span up to three groups (two for g >= 32); the first group holds the first
// b1 = g - (40T mod g) codes, a multiple of 8, so codes in the same octet share a group.
// x0 = (w & 0xFFFF) | ((w << 1) & 0xFFFF0000) puts (c0, c5), (c1, c6), (c2, c7) at bits 0, 3, 6
// of the two halves and x0 >> 9 puts (c3, c8), (c4, c9) at bits 0, 3.  A wave's 5 KB of
// output goes through LDS, five 1 KB store instructions.  Thread nfull = N / 40 writes the
// last N mod 40 codes one at a time.
template <bool THREE>
__global__ void __launch_bounds__(256) k_dqh3_ax1(const uint32_t* __restrict__ packed,
                                                  const unsigned short* __restrict__ delta,
                                                  const unsigned short* __restrict__ zero, int64_t N, int gshift,
                                                  __half* __restrict__ out) {
  __shared__ uint4 stage[4][320];
  const int lane = threadIdx.x & 63, wi = threadIdx.x >> 6;
  const int64_t T = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nfull = N / 40;
  const int64_t G = N >> gshift;
  const int g = 1 << gshift;
  if (nfull > 0) {
    const int64_t Tc = min(T, nfull - 1);  // threads past the end recompute the last chunk, unstored
    const uint4 wq = reinterpret_cast<const uint4*>(packed)[Tc];
    const int64_t base = 40 * Tc;
    const int64_t j0 = base >> gshift;
    const int b1 = g - (int)(base & (g - 1));
    constexpr int NG = THREE ? 3 : 2;
    unsigned zv[NG], dv[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int64_t j = min(j0 + k, G - 1);
      zv[k] = zero[j];
      dv[k] = delta[j];
    }
    float zd[NG], d24[NG], d21[NG], d18[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      zd[k] = hmul<0>(zv[k], dv[k]);
      d24[k] = hscale<0>(dv[k], p2(24));
      d21[k] = hscale<0>(dv[k], p2(21));
      d18[k] = hscale<0>(dv[k], p2(18));
    }
    const unsigned wa[4] = {wq.x, wq.y, wq.z, wq.w};
    unsigned r[20];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const unsigned w = wa[v];
      const unsigned x0 = (w & 0x0000FFFFu) | ((w << 1) & 0xFFFF0000u);
      const unsigned x1 = x0 >> 9;
      const unsigned p[5] = {x0 & 0x00070007u, x0 & 0x00380038u, x0 & 0x01C001C0u, x1 & 0x00070007u,
                             x1 & 0x00380038u};
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        const int q = 10 * v + k;  // code index inside the thread's 40
        // group of code q: 0 if q < b1, 1 if q < b1 + g, else 2 (b1 >= 8, octets share it)
        const int oct = q >> 3;
        const bool in0 = oct == 0 || 8 * oct < b1;
        const bool in1 = !THREE || 8 * oct < b1 + g;
        const int src = k % 5;  // pair register
        const int sel = k / 5;  // low half: c0..c4, high half: c5..c9
        const int pos = src % 3 == 0 ? 24 : (src % 3 == 1 ? 21 : 18);  // bit 0, 3 or 6 of the half
        const float* dsv = pos == 24 ? d24 : (pos == 21 ? d21 : d18);
        const float dsel = in0 ? dsv[0] : (in1 ? dsv[1] : dsv[NG - 1]);
        const float zsel = in0 ? zd[0] : (in1 ? zd[1] : zd[NG - 1]);
        const int dw = q / 2;  // output dword (two codes)
        if (sel == 0) {
          if (q % 2 == 0) put<0, true>(r[dw], p[src], dsel, zsel);
          else put<0, false>(r[dw], p[src], dsel, zsel);
        } else {
          if (q % 2 == 0) put<1, true>(r[dw], p[src], dsel, zsel);
          else put<1, false>(r[dw], p[src], dsel, zsel);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < 5; ++b) stage[wi][5 * lane + b] = make_uint4(r[4 * b], r[4 * b + 1], r[4 * b + 2], r[4 * b + 3]);
    __builtin_amdgcn_wave_barrier();
    const int64_t T0 = (int64_t)blockIdx.x * 256 + wi * 64;  // thread of lane 0
    uint4* dst = reinterpret_cast<uint4*>(out + 40 * T0);
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const int ch = lane + 64 * b;  // 16-byte piece of the wave's output, written by lane ch / 5
      if (T0 + ch / 5 < nfull) st_nt(dst + ch, stage[wi][ch]);
    }
  }
  if (T == nfull) {
    // ragged end: codes 40 nfull .. N - 1, one at a time
    for (int64_t i = 40 * nfull; i < N; ++i) {
      const unsigned w = packed[i / 10];
      const unsigned cde = (w >> (3 * (i % 10))) & 7u;
      const int64_t j = i >> gshift;
      const unsigned zz = zero[j], dd = delta[j];
      const unsigned rr = mixlo0(cde, hscale<0>(dd, p2(24)), hmul<0>(zz, dd));
      reinterpret_cast<unsigned short*>(out)[i] = (unsigned short)rr;
    }
  }
}

template <int NBITS, int AXIS>
hipError_t dispatch_meta(const uint8_t* packed, const void* delta, const void* zero, int meta, int64_t N,
                         int64_t M, int gshift, __half* out, hipStream_t st) {
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  if (meta == HQQ_META_F16) {
    const unsigned short* dh = reinterpret_cast<const unsigned short*>(delta);
    const unsigned short* zh = reinterpret_cast<const unsigned short*>(zero);
    if constexpr (NBITS == 3 && AXIS == 1) {
      const int64_t threads = N / 40 + 1;  // the last one writes the ragged end (if any)
      const dim3 grid((unsigned)((threads + 255) / 256));
      if (gshift == 4)
        hipLaunchKernelGGL((k_dqh3_ax1<true>), grid, dim3(256), 0, st, pk, dh, zh, N, gshift, out);
      else
        hipLaunchKernelGGL((k_dqh3_ax1<false>), grid, dim3(256), 0, st, pk, dh, zh, N, gshift, out);
      return hipGetLastError();
    } else if constexpr (NBITS != 3 && AXIS == 1) {
      // words per thread: 2 at 4-bit (more blocks, a shorter tail: 11008x4096 20.8 us against 22.2
      // at 4; stores alone take 15.1 us and loads alone 7.8 there, so reads and writes share HBM)
      constexpr int CPW = 32 / NBITS, U = NBITS == 4 ? 2 : 4;
      const int64_t nwords = N / CPW;
      int wshift = 0;
      while ((CPW << wshift) < (1 << gshift)) ++wshift;
      const dim3 grid((unsigned)((nwords + 256 * U - 1) / (256 * U)));
      hipLaunchKernelGGL((k_dqh_ax1<NBITS, U>), grid, dim3(256), 0, st, pk, dh, zh, nwords, wshift, out);
      return hipGetLastError();
    } else if constexpr (NBITS != 3 && AXIS == 0) {
      constexpr int CPW = 32 / NBITS, U = 8;
      if (M % CPW == 0) {
        const int64_t chunks = M / CPW;
        const int g = 1 << gshift;
        const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)((g + U - 1) / U));
        hipLaunchKernelGGL((k_dqh_ax0<NBITS, U>), grid, dim3(256), 0, st, pk,
                           reinterpret_cast<const uint4*>(delta), reinterpret_cast<const uint4*>(zero), chunks, g,
                           out);
        return hipGetLastError();
      }
    }
  }
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
