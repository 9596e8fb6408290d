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
