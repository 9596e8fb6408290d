// Helpers shared by the fused dequant-product kernels: vector types, streaming loads, the
// fp16-subnormal code unpack, operand-slot permutation, lane reductions and output stores.
#pragma once

#include "hqq_internal.h"

namespace hqq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load of packed codes (read once: non-temporal).
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ f16x2 as_h2(unsigned u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ unsigned as_u(f16x2 h) { return __builtin_bit_cast(unsigned, h); }

// Unpack masks.  Kept as plain constants: ALU inline assembly would hide its register writes
// from the compiler's hazard tracking (an in-flight MFMA still reads its source VGPRs).
struct Masks {
  unsigned lo, hi, magic;
};
__device__ __forceinline__ Masks make_masks() { return Masks{0x000F000Fu, 0x00F000F0u, 0x64006400u}; }
__device__ __forceinline__ unsigned and_or(unsigned a, unsigned mask, unsigned magic) { return (a & mask) | magic; }

// Eight 4-bit codes -> fp16 subnormals in the order [c0, c4, 16c1, 16c5, c2, c6, 16c3, 16c7],
// each scaled by 2^-24: a masked nibble in the low mantissa bits of a binary16 with a zero
// exponent field is exactly c * 2^-24 (c * 2^-20 for the high nibble of a byte).  One AND per
// pair; the dot-product units and the MFMA keep subnormal inputs, products and sums stay in
// fp32, and the 2^24 is applied once per group.
constexpr float kSubScale = 16777216.0f;       // 2^24
constexpr float kSubScaleInv = 5.9604645e-08f;  // 2^-24
__device__ __forceinline__ f16x8 unpack8_sub(unsigned d) {
  const unsigned d8 = d >> 8;
  const u32x4 r = {d & 0x000F000Fu, d & 0x00F000F0u, d8 & 0x000F000Fu, d8 & 0x00F000F0u};
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ f16x8 cat(const f16x2 (&p)[4]) {
  const u32x4 r = {as_u(p[0]), as_u(p[1]), as_u(p[2]), as_u(p[3])};
  return __builtin_bit_cast(f16x8, r);
}

// Natural order x[0..7] (as 4 dwords of fp16 pairs) -> [x0, x4, x1, x5, x2, x6, x3, x7].
__device__ __forceinline__ uint4 perm_slots(uint4 v) {
  // v_perm_b32(hi_src, lo_src, sel): selector bytes 0-3 pick lo_src bytes, 4-7 hi_src bytes.
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // x0 | x4 << 16
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // x1 | x5 << 16
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // x2 | x6
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // x3 | x7
  return o;
}

template <int L, typename T>
__device__ __forceinline__ T seg_sum_f(T v) {
  if constexpr (L >= 2) v = v + __builtin_amdgcn_update_dpp(T(0), v, 0xB1, 0xF, 0xF, false);
  if constexpr (L >= 4) v = v + __builtin_amdgcn_update_dpp(T(0), v, 0x4E, 0xF, 0xF, false);
  if constexpr (L >= 8) v = v + __builtin_amdgcn_update_dpp(T(0), v, 0x141, 0xF, 0xF, false);
  if constexpr (L >= 16) v = v + __builtin_amdgcn_update_dpp(T(0), v, 0x140, 0xF, 0xF, false);
  return v;
}

__device__ __forceinline__ int quarter_of(int h) { return h == 1 ? 2 : (h == 2 ? 1 : h); }

template <int OUT>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
  if constexpr (OUT == HQQ_OUT_F16)
    reinterpret_cast<__half*>(y)[idx] = __float2half_rn(v);
  else
    reinterpret_cast<float*>(y)[idx] = v;
}

// ---- Codes -> fp16 W_hat = fp16(c 2^-24 (d 2^24) - z d) in natural order (the mixed fp16/fp32
// FMA: the code is a masked fp16 subnormal, z d is exact in fp32; one rounding to fp32 and one
// to fp16).  Used where the weight tile is dequantised before the matrix units.
// Eight 4-bit codes of a word (natural order) -> fp16 W_hat pairs (c0,c1), (c2,c3), (c4,c5), (c6,c7).
// t0 = (c0, c4), t1 = 16 (c1, c5), t2 = (c2, c6), t3 = 16 (c3, c7) as fp16 subnormals.
__device__ __forceinline__ u32x4 wq8(unsigned w, float ds24, float ds20, float zd) {
  const unsigned u = w >> 8;
  const f16x2 h0 = as_h2(w & 0x000F000Fu), h1 = as_h2(w & 0x00F000F0u);
  const f16x2 h2 = as_h2(u & 0x000F000Fu), h3 = as_h2(u & 0x00F000F0u);
  const f16x2 p0 = {(_Float16)__builtin_fmaf((float)h0[0], ds24, -zd), (_Float16)__builtin_fmaf((float)h1[0], ds20, -zd)};
  const f16x2 p1 = {(_Float16)__builtin_fmaf((float)h2[0], ds24, -zd), (_Float16)__builtin_fmaf((float)h3[0], ds20, -zd)};
  const f16x2 p2 = {(_Float16)__builtin_fmaf((float)h0[1], ds24, -zd), (_Float16)__builtin_fmaf((float)h1[1], ds20, -zd)};
  const f16x2 p3 = {(_Float16)__builtin_fmaf((float)h2[1], ds24, -zd), (_Float16)__builtin_fmaf((float)h3[1], ds20, -zd)};
  return u32x4{as_u(p0), as_u(p1), as_u(p2), as_u(p3)};
}

// Sixteen 2-bit codes of a word (natural order) -> fp16 W_hat pairs: lo = (c0,c1) .. (c6,c7),
// hi = (c8,c9) .. (c14,c15).  The masks 3 << 2t on w and on w >> 8 give (c_t, c_t+8) and
// (c_t+4, c_t+12) as fp16 subnormals at 4^t 2^-24; ds[t] = d 2^24 / 4^t.
__device__ __forceinline__ void wq16_2b(unsigned w, const float (&ds)[4], float zd, u32x4& lo, u32x4& hi) {
  const unsigned u = w >> 8;
  f16x2 h[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    h[t] = as_h2(w & (0x00030003u << (2 * t)));
    h[4 + t] = as_h2(u & (0x00030003u << (2 * t)));
  }
  // pair q: element q >> 2 of h[a] and h[a + 1], a = 2 (q & 3).  Each half is written on its own,
  // which the compiler selects as one v_fma_mixlo/mixhi_f16 each (a two-element vector built at
  // once became v_fma_mix_f32 pairs and a v_cvt_pk_f16_f32)
  unsigned r[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int a = 2 * (q & 3), e = q >> 2;
    f16x2 p;
    p[0] = (_Float16)__builtin_fmaf((float)h[a][e], ds[a & 3], -zd);
    p[1] = (_Float16)__builtin_fmaf((float)h[a + 1][e], ds[(a + 1) & 3], -zd);
    r[q] = as_u(p);
  }
  lo = u32x4{r[0], r[1], r[2], r[3]};
  hi = u32x4{r[4], r[5], r[6], r[7]};
}

// Eight 3-bit codes in bits 0..23 of v (natural order) -> fp16 W_hat pairs (c0,c1) .. (c6,c7):
// spread to two halves (codes 4..7 move up by 4 bits), the masks 7 << 3t give (c_t, c_t+4) at
// 8^t 2^-24 for t < 3 and the fourth pair after a 9-bit shift.
__device__ __forceinline__ u32x4 wq8_3b(unsigned v, float ds24, float ds21, float ds18, float zd) {
  const unsigned x0 = (v & 0x00000FFFu) | ((v << 4) & 0x0FFF0000u);
  const f16x2 h0 = as_h2(x0 & 0x00070007u), h1 = as_h2(x0 & 0x00380038u), h2 = as_h2(x0 & 0x01C001C0u),
              h3 = as_h2((x0 >> 9) & 0x00070007u);
  auto pr = [&](f16x2 a, float sa, f16x2 b, float sb, int e) {
    return as_u(f16x2{(_Float16)__builtin_fmaf((float)a[e], sa, -zd), (_Float16)__builtin_fmaf((float)b[e], sb, -zd)});
  };
  return u32x4{pr(h0, ds24, h1, ds21, 0), pr(h2, ds18, h3, ds24, 0), pr(h0, ds24, h1, ds21, 1), pr(h2, ds18, h3, ds24, 1)};
}

// Thirty-two 3-bit codes starting at an even slot ph (<= 8) of w[0] and ending in w[3] -> fp16
// W_hat in natural order, o[b] = codes 8b .. 8b + 7; codes 0..15 take step d[0] and zero-step
// product zd[0], codes 16..31 d[1], zd[1].  Block b starts at slot o = ph + 8b: in word o / 10,
// which is b - 1 or b (b >= 1) depending on ph; it ends in the next word or (o >= 30, then
// o / 10 = 3 and 3 (o - 30) + 24 <= 30) in the same one.  A 64-bit window of two words (30-bit
// payloads) shifted by 3 (o mod 10) puts the block's 24 bits at bits 0..23.
__device__ __forceinline__ void decode32_3b(const unsigned (&w)[4], int ph, const float (&d)[2], const float (&zd)[2],
                                            u32x4 (&o)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bool up = b > 0 && ph >= 2 * b;
    const int i = up ? b : (b > 0 ? b - 1 : 0);
    const unsigned lo = up ? w[b] : w[b > 0 ? b - 1 : 0];
    const unsigned hi = up ? (b < 3 ? w[b + 1] : 0u) : w[b > 0 ? b : 1];
    const int sh = 3 * (ph + 8 * b - 10 * i);
    const unsigned v = (unsigned)((((uint64_t)hi << 30) | (lo & 0x3FFFFFFFu)) >> sh);
    const int h = b >> 1;
    o[b] = wq8_3b(v, d[h] * 16777216.0f, d[h] * 2097152.0f, d[h] * 262144.0f, zd[h]);
  }
}

// Sum of the eight fp16 values of a 16-byte block (fp32 accumulation of x * 1).
__device__ __forceinline__ float block_sum8(const unsigned (&r4)[4]) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  float part = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) part = __builtin_amdgcn_fdot2(as_h2(r4[t]), one, part, false);
  return part;
}

// Sum over the 64 lanes of a wave (every lane gets the total): DPP inside rows of 16 lanes,
// then the rows pairwise (lane xor 16, xor 32).
__device__ __forceinline__ float wave_sum(float v) {
  v = seg_sum_f<16>(v);
  v = v + __shfl_xor(v, 16, 64);
  v = v + __shfl_xor(v, 32, 64);
  return v;
}

// Workgroup barrier for LDS hand-over only: waits for this wave's LDS operations, not for its
// global loads (the prefetched operands stay in flight; __syncthreads would drain them).  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace hqq
