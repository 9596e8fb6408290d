// Fused dequantise + product, 4-bit weights, fp16 activations, fp32 accumulation (page
// "HQQ 算法解读", section "从压缩文件到一次前向": unpack, (q - zero) * scale, x @ W_hat^T).
//
// Three kernels:
//   k_gemv_valu  batch 1-2: each wave streams whole rows (1 KB of one row per load instruction)
//                and forms the group sums with v_dot2_f32_f16 on exact codes;
//   k_gemv_mf    batch 3-8 (and 1-2 with rows longer than 16384 codes): v_mfma_f32_16x16x32_f16,
//                the packed rows staged through LDS so that the global loads stay row-contiguous;
//   k_gemm       batch > 8 without a workspace: an MFMA GEMM on fp16 W_hat tiles.
//
// MFMA operand layout: the weight tile is the B operand (16 output rows n per tile,
// n = lane % 16), the activations are the A operand (16 rows m, m = lane % 16), and lane
// (h = lane / 16, r) of the result holds row m = 4h + r, column n.  A load instruction whose
// lanes span 16 rows reads the weight stream at half the rate of one that reads 1 KB of one row
// (the rows are pages apart), hence the LDS staging.  Lane group h of the B operand holds codes
// 32h .. 32h + 31 of a 128-code chunk.  With groups of 128 the chunk is one group and m is the
// batch row.  With groups of 64 each MFMA sums 16 codes of each of the chunk's two groups, so A
// row m < 8 carries batch row m against the first group's k slots (zeros against the second's)
// and row 8 + m batch row m against the second's: result rows 0-7 are the first group's
// partial sums, rows 8-15 the second's, and each group's delta and zero are applied once on
// them, with no result row left for padding at batch 8.
//
// Code unpack (fp16 subnormals): for a dword of eight 4-bit codes c0..c7, (d & 0x000F000F) is
// the fp16 pair (c0, c4) * 2^-24 and (d & 0x00F000F0) the pair (16 c1, 16 c5) * 2^-24, the same
// on d >> 8; the dot-product units and the MFMA keep subnormal inputs.  The operand order within
// a lane's eight k slots is therefore [0, 4, 1, 5, 2, 6, 3, 7] with a factor 16 on the odd
// codes; the activations are staged in the same order with 1/16 on the odd codes.  q stays
// exact; the group's metadata is applied on the fp32 partial: acc += delta * (P - z * sum_k x_k),
// with the 2^24 folded into the step and the zero.
// The batch > 8 GEMM dequantises its tile to fp16 W_hat = (q - z) * delta first (the plain
// "dequantise then matmul" of the page, with fp32 accumulation).

#include <type_traits>

#include "hqq_gemv_common.h"

namespace hqq {
namespace {

// ------------------------------------------------------------------------------------------
// GEMV, batch 3..8, on the MFMA unit with the whole pipeline in one block.
// Block = W waves (8, or 16 for rows past 8192 codes) on RB = 16 SPB weight rows; K is walked in
// segments of 128 W codes and wave w always takes the 128-code chunk w of a segment, for every
// strip of the block (the A fragments it reads from LDS serve all strips).  Per segment the
// block stages, double buffered in LDS: x in the MFMA operand order (1/16 on the odd codes)
// with the per-group sums of x, the packed rows (each load instruction reads 1 KB of one or two
// rows; the operand layout would put 16 rows, 16 pages, into each), and the rows' steps and
// zeros.  The loads run two segments ahead in registers; one LDS-only barrier per segment.  At
// the end the W waves' partial sums of each output are added in wave order (deterministic).
// ------------------------------------------------------------------------------------------
// Block geometry for W waves: one 128-code chunk of a segment per wave.
template <int W>
struct MfGeom {
  static constexpr int ks = 128 * W;            // codes per segment
  static constexpr int ksp = ks + 8;            // LDS row stride of x (halves): rows in different banks
  static constexpr int wrb = ks / 2 + 16;       // LDS row stride of the packed codes (bytes)
  static constexpr int pieces = ks / 32;        // 16-byte pieces of one row's segment of codes
  static constexpr int rows_per_wave = 16 / W;  // rows of a strip each wave loads per segment
  static_assert(pieces * rows_per_wave == 64 && 16 % W == 0, "a wave loads whole row segments");
};

// Batch rows of the per-group sums of x, padded with zeros (8 with groups of 64: a lane reads the
// sums of batch rows 0-3 or 4-7).
__host__ __device__ constexpr int mf_bp(int B, int GS) { return GS == 64 ? 8 : (B + 3) & ~3; }
// LDS bytes of one stage (x, sums of x, codes, metadata) and of the kernel (two stages, and with
// groups of 64 a row of zeros that the A rows read against the other group's codes).
__host__ __device__ constexpr int mf_stage_bytes(int B, int GS, int SPB, int W) {
  return B * (128 * W + 8) * 2 + (128 * W / GS) * mf_bp(B, GS) * 4 + 16 * SPB * (64 * W + 16) +
         16 * SPB * (2 * (128 * W / GS) + 4) * 4;
}
__host__ __device__ constexpr int mf_lds_bytes(int B, int GS, int SPB, int W) {
  return 2 * mf_stage_bytes(B, GS, SPB, W) + (GS == 64 ? 128 * W * 2 : 0);
}

template <int B, int GS, int SPB, int NSEG, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_mf(const uint8_t* __restrict__ packed,
                                                   const __half* __restrict__ delta,
                                                   const __half* __restrict__ zero, int64_t N, int64_t K,
                                                   const __half* __restrict__ x, void* __restrict__ y,
                                                   int out_dtype) {
  static_assert(B >= 1 && B <= 8 && (GS == 64 || GS == 128) && (SPB == 1 || SPB == 2), "shape");
  constexpr int kMfWaves = W, kMfKS = MfGeom<W>::ks, kMfKSP = MfGeom<W>::ksp, kMfWRB = MfGeom<W>::wrb;
  constexpr int kMfPieces = MfGeom<W>::pieces, kMfRowsPerWave = MfGeom<W>::rows_per_wave;
  constexpr int NT = 64 * kMfWaves, RB = 16 * SPB;
  constexpr int GPS = kMfKS / GS;          // groups per segment and row
  constexpr int XB = B * (kMfKS / 8);      // 16-byte blocks of x per segment
  constexpr int XR = (XB + NT - 1) / NT;   // of them per thread
  constexpr int MW = GS == 64 ? 2 : 1;     // groups per metadata load (4 or 2 bytes)
  constexpr int ML = RB * GPS / MW;        // metadata loads per array and segment
  constexpr int BP = mf_bp(B, GS);         // batch rows of the x sums, padded with zeros
  constexpr int MLR = 2 * GPS + 4;         // LDS row stride of the metadata (floats): 16-byte reads of 8
                                           // consecutive rows fall in distinct banks
  static_assert(ML <= NT, "one step and one zero load per thread");
  constexpr int STAGE = mf_stage_bytes(B, GS, SPB, W);
  extern __shared__ __align__(16) uint8_t lds_raw[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 4, nl = lane & 15;
  const int arow = nl < B ? nl : 0;  // A rows >= B only feed outputs that are never stored
  const int64_t n0 = (int64_t)blockIdx.x * RB;
  const int64_t gpr = K / GS;
  const int64_t nchunks = K / 128;
  // segments: a compile-time count (1..8) makes the pipeline straight-line code, so the memory
  // counter waits name exactly the loads about to be staged; 0 = a run-time loop (longer rows)
  const int nseg = NSEG > 0 ? NSEG : (int)((K + kMfKS - 1) / kMfKS);

  // stage layout
  auto xs_of = [&](int buf) { return reinterpret_cast<_Float16*>(lds_raw + buf * STAGE); };
  // per group of the segment the sums of x over its codes, [GPS][BP]; per row and group the
  // step times 2^24 and minus the zero times 2^-24 (fp32, converted once at staging), [RB][MLR]
  auto sx_of = [&](int buf) { return reinterpret_cast<float*>(lds_raw + buf * STAGE + B * kMfKSP * 2); };
  auto wl_of = [&](int buf) { return lds_raw + buf * STAGE + B * kMfKSP * 2 + GPS * BP * 4; };
  auto ml_of = [&](int buf) {
    return reinterpret_cast<float*>(lds_raw + buf * STAGE + B * kMfKSP * 2 + GPS * BP * 4 + RB * kMfWRB);
  };

  // ---- loads of one segment into a register set (unconditional, clamped indexes: a load under
  //      a branch makes the compiler wait for it at the join)
  struct Regs {
    uint4 xr[XR];
    uint4 wr[SPB];
    unsigned md, mz;  // steps and zeros of one to two groups (fp16)
  };
  auto load_seg = [&](int sg, Regs& r) {
    const int64_t kb0 = (int64_t)sg * kMfKS;
    const int valid = (int)((K - kb0 < kMfKS) ? (K - kb0) : kMfKS);  // codes of the segment (a multiple of 128)
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = min(tid + NT * j, XB - 1);
      const int m = idx / (kMfKS / 8), kb = min(idx % (kMfKS / 8), valid / 8 - 1);
      r.xr[j] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + kb0 + 8 * kb);
    }
#pragma unroll
    for (int j = 0; j < SPB; ++j) {  // each wave takes 16 / kMfWaves rows of the strip
      const int row = kMfRowsPerWave * wave + lane / kMfPieces + 16 * j;
      const int piece = min(lane % kMfPieces, valid / 32 - 1);  // 16-byte pieces of the row's segment
      r.wr[j] = ld_stream16(packed + (n0 + row) * (K / 2) + kb0 / 2 + 16 * piece);
    }
    {
      const int i = min(tid, ML - 1);
      const int row = i / (GPS / MW), pc = min(i % (GPS / MW), valid / (GS * MW) - 1);  // valid % 128 == 0
      const int64_t gi = (n0 + row) * gpr + kb0 / GS + (int64_t)MW * pc;
      r.md = MW == 2 ? *reinterpret_cast<const unsigned*>(delta + gi) : (unsigned)__half_as_ushort(delta[gi]);
      r.mz = MW == 2 ? *reinterpret_cast<const unsigned*>(zero + gi) : (unsigned)__half_as_ushort(zero[gi]);
    }
  };
  // ---- a register set -> LDS stage `buf`
  auto stage_seg = [&](int sg, int buf, const Regs& r) {
    const int64_t kb0 = (int64_t)sg * kMfKS;
    const int valid = (int)((K - kb0 < kMfKS) ? (K - kb0) : kMfKS);
    _Float16* xs = xs_of(buf);
    float* sx = sx_of(buf);
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = tid + NT * j;
      if (idx < XB) {  // uniform per 64-lane run: a group's GS/8 blocks stay in one run
        const int m = idx / (kMfKS / 8), kb = idx % (kMfKS / 8);
        const uint4 raw = r.xr[j];
        const unsigned r4[4] = {raw.x, raw.y, raw.z, raw.w};
        float part = block_sum8(r4);
        uint4 o = perm_slots(raw);
        o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        *reinterpret_cast<uint4*>(xs + m * kMfKSP + 8 * kb) = o;
        part = seg_sum_f<GS / 8>(part);
        if ((kb % (GS / 8)) == 0 && 8 * kb < valid) sx[(kb / (GS / 8)) * BP + m] = part;
      }
    }
    uint8_t* wl = wl_of(buf);
#pragma unroll
    for (int j = 0; j < SPB; ++j)
      *reinterpret_cast<uint4*>(wl + (kMfRowsPerWave * wave + lane / kMfPieces + 16 * j) * kMfWRB +
                                16 * (lane % kMfPieces)) = r.wr[j];
    if (tid < ML) {
      // P = 2^-24 sum x q (subnormal codes): the step is scaled up and the zero down by 2^24 (exact)
      const int row = tid / (GPS / MW), pc = tid % (GPS / MW);
      float* ml = ml_of(buf) + row * MLR + 2 * MW * pc;
      const float d0 = __half2float(__ushort_as_half((unsigned short)r.md)) * kSubScale;
      const float z0 = __half2float(__ushort_as_half((unsigned short)r.mz)) * -kSubScaleInv;
      if (MW == 2) {
        const float d1 = __half2float(__ushort_as_half((unsigned short)(r.md >> 16))) * kSubScale;
        const float z1 = __half2float(__ushort_as_half((unsigned short)(r.mz >> 16))) * -kSubScaleInv;
        *reinterpret_cast<f32x4*>(ml) = f32x4{d0, z0, d1, z1};
      } else {
        *reinterpret_cast<float2*>(ml) = make_float2(d0, z0);
      }
    }
  };

  f32x4 acc[SPB];
#pragma unroll
  for (int sp = 0; sp < SPB; ++sp) acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two register sets, each always holding a segment in flight: iteration `cur` first stages
  // segment cur + 1 (requested two iterations earlier) into the stage the block finished
  // reading an iteration ago, refills that register set with segment cur + 3, then multiplies
  // segment cur; one LDS-only barrier per iteration.
  if constexpr (BP > B) {  // padded batch rows of the x sums stay zero (staging never writes them)
    for (int i = tid; i < 2 * GPS * (BP - B); i += NT) {
      const int b = i / (GPS * (BP - B)), rem = i % (GPS * (BP - B));
      sx_of(b)[(rem / (BP - B)) * BP + B + rem % (BP - B)] = 0.f;
    }
  }
  const _Float16* zrow = reinterpret_cast<const _Float16*>(lds_raw + 2 * STAGE);  // GS == 64: kMfKS zeros
  if constexpr (GS == 64) {
    static_assert(kMfKS / 2 == NT, "one dword of the zero row per thread");
    reinterpret_cast<unsigned*>(lds_raw + 2 * STAGE)[tid] = 0u;
  }
  // GS == 64: A row m < 8 is batch row m against the first group of a chunk, row 8 + m batch row m
  // against the second; the lane supplies x where its k slots hold codes of that row's group and
  // zeros (the zero row) elsewhere and past the batch
  const bool xact = ((nl < 8) == (h < 2)) && (nl & 7) < B;
  Regs rs[2];
  load_seg(0, rs[0]);
  if (NSEG != 1) load_seg(min(1, nseg - 1), rs[1]);
  stage_seg(0, 0, rs[0]);
  if (NSEG == 0 || NSEG > 2) load_seg(min(2, nseg - 1), rs[0]);
  lds_barrier();
  // one segment: stage `cur` + 1 (requested two segments earlier) into the other stage, refill
  // that register set with `cur` + 3, multiply `cur`; one LDS-only barrier
  auto segment = [&](const int cur, auto bufc) {
    constexpr int buf = decltype(bufc)::value;  // segment cur lives in stage cur % 2
    if (cur + 1 < nseg) stage_seg(cur + 1, buf ^ 1, rs[buf ^ 1]);  // waits only for those loads
    if (NSEG == 0 || cur + 3 < NSEG) load_seg(min(cur + 3, nseg - 1), rs[buf ^ 1]);
    const int64_t c = (int64_t)cur * kMfWaves + wave;  // this wave's chunk
    if (c < nchunks) {
      const _Float16* xs = xs_of(buf);
      const float* sx = sx_of(buf);
      const uint8_t* wl = wl_of(buf);
      const float* ml = ml_of(buf);
      if constexpr (GS == 64) {
        // lane group h holds codes 32 h .. 32 h + 31 of the chunk: lane groups 0-1 the first group
        // (64 codes), 2-3 the second, so each MFMA sums 16 codes of each group, and result rows
        // 0-7 (lane groups 0-1) are the first group's partial sums for batch rows 0-7, rows 8-15
        // (lane groups 2-3) the second group's
        const _Float16* xa = (xact ? xs + (nl & 7) * kMfKSP : zrow) + wave * 128 + 32 * h;
        f16x8 A[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) A[t] = *reinterpret_cast<const f16x8*>(xa + 8 * t);
        // sums of x of this lane's group and batch rows 4 (h & 1) .. + 3
        const f32x4 sxv = *reinterpret_cast<const f32x4*>(sx + (2 * wave + (h >> 1)) * BP + 4 * (h & 1));
#pragma unroll
        for (int sp = 0; sp < SPB; ++sp) {
          const int row = 16 * sp + nl;
          const uint4 v = *reinterpret_cast<const uint4*>(wl + row * kMfWRB + wave * 64 + h * 16);
          const unsigned dd[4] = {v.x, v.y, v.z, v.w};
          f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], unpack8_sub(dd[t]), P, 0, 0, 0);
          const float2 md = *reinterpret_cast<const float2*>(ml + row * MLR + 4 * wave + 2 * (h >> 1));  // d, -z
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[sp][r] = fmaf(md.x, fmaf(md.y, sxv[r], P[r]), acc[sp][r]);
        }
      } else {  // GS == 128: the chunk is one group; lane group h holds codes 32 h .. 32 h + 31
        f16x8 A[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          A[t] = *reinterpret_cast<const f16x8*>(xs + arow * kMfKSP + wave * 128 + h * 32 + t * 8);
        const int hq = 4 * h < BP ? 4 * h : 0;
        f32x4 sxv = *reinterpret_cast<const f32x4*>(sx + wave * BP + hq);
        if (4 * h >= BP) sxv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < SPB; ++sp) {
          const int row = 16 * sp + nl;
          const uint4 v = *reinterpret_cast<const uint4*>(wl + row * kMfWRB + wave * 64 + h * 16);
          const unsigned dd[4] = {v.x, v.y, v.z, v.w};
          f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], unpack8_sub(dd[t]), P, 0, 0, 0);
          const float2 md = *reinterpret_cast<const float2*>(ml + row * MLR + 2 * wave);  // d, -z
#pragma unroll
          for (int r = 0; r < (B < 4 ? B : 4); ++r) acc[sp][r] = fmaf(md.x, fmaf(md.y, sxv[r], P[r]), acc[sp][r]);
        }
      }
    }
    lds_barrier();
  };
  if constexpr (NSEG > 0) {
#pragma unroll
    for (int cur = 0; cur < NSEG; ++cur) {
      if (cur % 2 == 0)
        segment(cur, std::integral_constant<int, 0>{});
      else
        segment(cur, std::integral_constant<int, 1>{});
    }
  } else {
    for (int cur = 0; cur < nseg; cur += 2) {
      segment(cur, std::integral_constant<int, 0>{});
      if (cur + 1 < nseg) segment(cur + 1, std::integral_constant<int, 1>{});
    }
  }
  // ---- the W waves' partial sums of each output, added in wave order (stage memory reused)
  float* red = reinterpret_cast<float*>(lds_raw);  // [SPB][W waves][B][16]
  if constexpr (GS == 64) {
    // first groups' sums (lanes 0-31) plus second groups' (lanes 32-63): one swap of the pair
    // (r, r + 1) leaves row r's total in lanes 0-31 and row r + 1's in lanes 32-63, so lane
    // (h, n) holds batch row 4 (h & 1) + r + (h >> 1)
#pragma unroll
    for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        // (__float_as_uint on the element values: a bit cast of a vector element lvalue reads
        // element 0 with this compiler)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[sp][r]), __float_as_uint(acc[sp][r + 1]),
                                                         false, false);
        const float t = __uint_as_float((unsigned)sw[0]) + __uint_as_float((unsigned)sw[1]);
        const int m = 4 * (h & 1) + r + (h >> 1);
        if (m < B) red[((sp * kMfWaves + wave) * B + m) * 16 + nl] = t;
      }
  } else {
#pragma unroll
    for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
      for (int r = 0; r < (B < 4 ? B : 4); ++r) {
        const int m = 4 * h + r;
        if (m < B) red[((sp * kMfWaves + wave) * B + m) * 16 + nl] = acc[sp][r];
      }
  }
  lds_barrier();
  if (tid < SPB * B * 16) {
    const int sp = tid / (B * 16), m = (tid / 16) % B, col = tid % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kMfWaves; ++w) sum += red[((sp * kMfWaves + w) * B + m) * 16 + col];
    if (out_dtype == HQQ_OUT_F16)
      store_y<HQQ_OUT_F16>(y, (int64_t)m * N + n0 + 16 * sp + col, sum);
    else
      store_y<HQQ_OUT_F32>(y, (int64_t)m * N + n0 + 16 * sp + col, sum);
  }
}

// ------------------------------------------------------------------------------------------
// GEMV on the vector ALUs, batch B <= 2.  Each wave streams whole rows: lane l takes the
// 32-code chunks c = l + 64 j of a row, so one load instruction reads 1 KB of one row.  Per
// chunk the lane forms P = sum x_k q_k with v_dot2_f32_f16 on exact codes and applies the
// group's step and zero on the fp32 partial, acc += delta * (P - z * sum_k x_k); row results
// are reduced over the wave's lanes with a fixed tree.
//
// Pipelining: wave gw of the grid takes exactly R consecutive rows, n = gw R + k, so each wave
// streams one contiguous run of R rows (measured at 8192 x 8192, batch 1: 7.77 us, against 8.00
// with the rows of a wave N / R apart and 8.04 with a block's waves on neighbouring rows at each
// step).  D rows are in flight per wave:
// row k + D is requested as soon as row k has been multiplied.  Everything a wave does is
// straight-line code: loads are unconditional (a chunk index past the row's end is clamped
// and its contribution selected away), so the compiler's memory-counter waits only ever wait
// for the row about to be used, never for the whole pipeline.
//
// The activations are staged once per block in LDS in the unpack order (1/16 on the odd
// codes) with the per-chunk sums of x; with XREG the lane then keeps its own chunks of x in
// registers for all its rows (no LDS traffic in the row loop).
// ------------------------------------------------------------------------------------------
constexpr int kVWaves = 4;  // waves per block of the VALU GEMV

// LDS bytes of the VALU GEMV: per-chunk sums of x, then x in 16-byte blocks.
__host__ __device__ constexpr int64_t valu_lds_bytes(int B, int64_t K) {
  return ((B * (K / 32) + 3) & ~int64_t(3)) * 4 + (int64_t)B * K * 2;
}

template <int B, int JMAX, int R, int D = (R < 2 ? R : 2), int W = kVWaves>
__global__ void __launch_bounds__(64 * W) k_gemv_valu(const uint8_t* __restrict__ packed,
                                                           const __half* __restrict__ delta,
                                                           const __half* __restrict__ zero, int64_t N, int64_t K,
                                                           int gs_log2, int out_dtype, const __half* __restrict__ x,
                                                           void* __restrict__ y) {
  static_assert(D >= 1 && D <= R, "rows in flight (D) must be within the wave's R rows");
  constexpr bool XREG = B * JMAX <= 4;         // x chunks held in registers
  constexpr int NT = 64 * W;                   // W waves per block
  extern __shared__ float lds[];
  const int nch = (int)(K / 32);               // 32-code chunks per row
  float* sxc = lds;                            // [B][nch] sum of x over each chunk
  uint4* xs = reinterpret_cast<uint4*>(sxc + ((B * nch + 3) & ~3));  // [B][4][nch] 16-byte blocks
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t gpr = K >> gs_log2;            // groups per row
  const int cshift = gs_log2 - 5;              // chunk -> group within the row
  const int64_t TW = 1;                                 // row step within a wave
  const int64_t gw = ((int64_t)blockIdx.x * W + wave) * R;  // the wave's first row

  // 1. this thread's 16-byte blocks of x (a block past the end re-reads the last one)
  constexpr int XR = (B * 64 * JMAX * 4 + NT - 1) / NT;
  const int nxb = B * nch * 4;
  uint4 xr[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = min(tid + NT * i, nxb - 1);
    xr[i] = *reinterpret_cast<const uint4*>(x + 8 * idx);  // x is [B][K] contiguous
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the weight stream

  // 2. the first D rows of this wave, in flight
  uint4 wv[D][JMAX];
  unsigned dmv[D][JMAX], zmv[D][JMAX];  // 32 bits each: two loads never share a register
  auto issue = [&](int s, int64_t n) {
    const uint8_t* wrow = packed + n * (K / 2);
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      wv[s][j] = ld_stream16(wrow + 16 * c);
      const int64_t gi = n * gpr + (c >> cshift);
      dmv[s][j] = __half_as_ushort(delta[gi]);
      zmv[s][j] = __half_as_ushort(zero[gi]);
    }
  };
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, gw + s * TW);

  // 3. stage x: 16-byte block t of chunk c of batch row m at xs[(m * 4 + t) * nch + c], unpack
  //    order, 1/16 on the odd codes; chunk sums of the unscaled x.  Clamped indexes rewrite the
  //    last block with the same value.
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = min(tid + NT * i, nxb - 1);
    const int m = idx / (nch * 4), rem = idx % (nch * 4), c = rem / 4, t = rem % 4;
    const uint4 raw = xr[i];
    const unsigned r4[4] = {raw.x, raw.y, raw.z, raw.w};
    float part = block_sum8(r4);
    uint4 o = perm_slots(raw);
    o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
    o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
    xs[(m * 4 + t) * nch + c] = o;
    part = seg_sum_f<4>(part);  // the 4 lanes of a chunk are consecutive and active together
    if (t == 0) sxc[m * nch + c] = part;
  }
  lds_barrier();  // LDS hand-over; the weight loads stay in flight
  f16x2 xq[XREG ? B : 1][XREG ? JMAX : 1][16];
  float sxr[B][JMAX];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      if constexpr (XREG) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 v = xs[(b * 4 + t) * nch + c];
          xq[b][j][4 * t + 0] = as_h2(v.x);
          xq[b][j][4 * t + 1] = as_h2(v.y);
          xq[b][j][4 * t + 2] = as_h2(v.z);
          xq[b][j][4 * t + 3] = as_h2(v.w);
        }
      }
      sxr[b][j] = sxc[b * nch + c];
    }

  // 4. rows: multiply row k, then request row k + D into the freed slot
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int s = k % D;
    const int64_t n = gw + k * TW;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      const bool valid = lane + 64 * j < nch;
      const unsigned dw[4] = {wv[s][j].x, wv[s][j].y, wv[s][j].z, wv[s][j].w};
      f16x2 q[16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 u = __builtin_bit_cast(u32x4, unpack8_sub(dw[t]));
#pragma unroll
        for (int e = 0; e < 4; ++e) q[4 * t + e] = as_h2(u[e]);
      }
      // codes are 2^-24 * q (subnormal unpack): the step is scaled up and the zero down
      const float dl = valid ? __half2float(__ushort_as_half((unsigned short)dmv[s][j])) * kSubScale : 0.f;
      const float zz = __half2float(__ushort_as_half((unsigned short)zmv[s][j])) * kSubScaleInv;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float P = 0.f;
        if constexpr (XREG) {
#pragma unroll
          for (int e = 0; e < 16; ++e) P = __builtin_amdgcn_fdot2(xq[b][j][e], q[e], P, false);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint4 xv = xs[(b * 4 + t) * nch + c];
            const unsigned xu[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) P = __builtin_amdgcn_fdot2(as_h2(xu[e]), q[4 * t + e], P, false);
          }
        }
        acc[b] = fmaf(dl, fmaf(-zz, sxr[b][j], P), acc[b]);
      }
    }
    if (k + D < R) issue(s, gw + (k + D) * TW);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum(acc[b]);
      if (lane == 0) {
        if (out_dtype == HQQ_OUT_F16)
          store_y<HQQ_OUT_F16>(y, (int64_t)b * N + n, v);
        else
          store_y<HQQ_OUT_F32>(y, (int64_t)b * N + n, v);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// GEMM, batch > 8.  Block = 4 waves, tile 128 batch rows x 64 output rows; wave w owns the
// output rows n0 + 16w .. +15 and all eight 16-row batch tiles.  The 128-code chunks of K are
// software-pipelined: the block's x tile for chunk c+1 is loaded into registers while chunk c
// is multiplied out of LDS, and each wave's packed weights run one chunk ahead.  Each wave
// dequantises its own weight rows to fp16 W_hat straight into the B-operand layout, with the
// codes unpacked in natural k order, so x is staged unchanged.
// ------------------------------------------------------------------------------------------
constexpr int kGemmM = 128;
constexpr int kGemmDepth = 4;  // chunks of 128 codes in flight per wave
constexpr int kXRow = 128 + 8;  // LDS row stride (halves) of the x tile

// Eight 4-bit codes -> fp16 pairs (c0,c1), (c2,c3), (c4,c5), (c6,c7), exact.
__device__ __forceinline__ void unpack8_natural(unsigned d, const Masks& mk, f16x2 (&p)[4]) {
  const unsigned d4 = d >> 4;  // high nibbles moved to the low nibble of each byte
  const f16x2 off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  // v_perm_b32: bytes 0-3 of the 64-bit {d4:d} pick d, 4-7 pick d4; byte b of d holds
  // c(2b) in its low nibble, byte b of d4 holds c(2b+1)
  p[0] = as_h2(and_or(__builtin_amdgcn_perm(d4, d, 0x0C040C00u), mk.lo, mk.magic)) + off;
  p[1] = as_h2(and_or(__builtin_amdgcn_perm(d4, d, 0x0C050C01u), mk.lo, mk.magic)) + off;
  p[2] = as_h2(and_or(__builtin_amdgcn_perm(d4, d, 0x0C060C02u), mk.lo, mk.magic)) + off;
  p[3] = as_h2(and_or(__builtin_amdgcn_perm(d4, d, 0x0C070C03u), mk.lo, mk.magic)) + off;
}

template <int GS, int OUT>
__global__ void __launch_bounds__(256) k_gemm(const uint8_t* __restrict__ packed, const __half* __restrict__ delta,
                                              const __half* __restrict__ zero, int64_t N, int64_t K,
                                              const __half* __restrict__ x, int64_t batch, void* __restrict__ y) {
  __shared__ _Float16 xt[kGemmM * kXRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 4, nl = lane & 15;
  const int64_t m0 = (int64_t)blockIdx.x * kGemmM;
  const int64_t nrow0 = (int64_t)blockIdx.y * 64 + wave * 16;
  // N is a multiple of 16: a wave's 16 rows are all inside or all outside; an outside wave
  // still stages its share of x and meets every barrier, it reads row nl and stores nothing.
  const bool wvalid = nrow0 < N;
  const int64_t n = wvalid ? nrow0 + nl : nl;
  const int64_t gpr = K / GS;
  const uint8_t* wrow = packed + n * (K / 2);
  const __half* drow = delta + n * gpr;
  const __half* zrow = zero + n * gpr;
  const int qh = quarter_of(h);
  const Masks mk = make_masks();

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x tile staging: thread -> 8 blocks of 8 halves (rows tid/16 + 16j, block tid%16).  Batch
  // rows past the end read the last row (unconditional loads: a load under a branch makes the
  // compiler wait for it at the join); their outputs are never stored.
  const int xr_row = tid >> 4, xr_kb = tid & 15;
  const __half* xrow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xrow[j] = x + min(m0 + xr_row + 16 * j, batch - 1) * K + 8 * xr_kb;
  // the chunk's packed codes and its groups' step and zero (two groups per chunk at g = 64)
  auto load_meta = [&](int64_t c, unsigned& dmw, unsigned& zmw) {
    if constexpr (GS == 64) {
      dmw = *reinterpret_cast<const unsigned*>(drow + 2 * c);
      zmw = *reinterpret_cast<const unsigned*>(zrow + 2 * c);
    } else {
      dmw = __half_as_ushort(drow[c]);
      zmw = __half_as_ushort(zrow[c]);
    }
  };
  const int64_t nchunks = K / 128;
  // Chunks c + 1 .. c + kGemmDepth - 1 are in flight (registers) while chunk c is multiplied:
  // the loop is unrolled by the depth so that every slot index is a constant.  Loads are
  // unconditional; chunk indexes past the end are clamped (the tail reloads the last chunk).
  u32x4 xb[kGemmDepth][8];  // native vector type: an array of the uint4 struct went to scratch
  u32x4 vb[kGemmDepth];
  unsigned db[kGemmDepth], zb[kGemmDepth];
#pragma unroll
  for (int sl = 0; sl < kGemmDepth; ++sl) {
    const int64_t c = sl < nchunks ? sl : nchunks - 1;
    vb[sl] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + c * 64 + h * 16));
    load_meta(c, db[sl], zb[sl]);
#pragma unroll
    for (int j = 0; j < 8; ++j) xb[sl][j] = *reinterpret_cast<const u32x4*>(xrow[j] + c * 128);
  }
  for (int64_t cb = 0; cb < nchunks; cb += kGemmDepth) {
#pragma unroll
    for (int sl = 0; sl < kGemmDepth; ++sl) {
      const int64_t c = cb + sl;
      // publish chunk c's x tile, take its codes and metadata, refill the slot with c + depth.
      // A chunk past the end (the last round of the unrolled loop) gets a zero step, so its
      // W_hat is 0 and it adds nothing: no branch, so the memory-counter waits stay exact.
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(xt + (xr_row + 16 * j) * kXRow + 8 * xr_kb) = xb[sl][j];
      const uint4 v = make_uint4(vb[sl][0], vb[sl][1], vb[sl][2], vb[sl][3]);
      const unsigned dmw = c < nchunks ? db[sl] : 0u, zmw = zb[sl];
      {
        const int64_t cn = c + kGemmDepth < nchunks ? c + kGemmDepth : nchunks - 1;
        vb[sl] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + cn * 64 + h * 16));
        load_meta(cn, db[sl], zb[sl]);
#pragma unroll
        for (int j = 0; j < 8; ++j) xb[sl][j] = *reinterpret_cast<const u32x4*>(xrow[j] + cn * 128);
      }
      // weights of chunk c -> fp16 W_hat in the B-operand layout (natural k order)
      f16x8 Bop[4];
      int kofs[4];
      if constexpr (GS == 64) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
        const unsigned gd[4] = {s0[0], s1[0], s0[1], s1[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gg = j >> 1, s = j & 1;
          const _Float16 dl = __builtin_bit_cast(_Float16, (unsigned short)(dmw >> (16 * gg)));
          const _Float16 zz = __builtin_bit_cast(_Float16, (unsigned short)(zmw >> (16 * gg)));
          const f16x2 z1 = {zz, zz}, d1 = {dl, dl};
          f16x2 p[4];
          unpack8_natural(gd[j], mk, p);
#pragma unroll
          for (int u = 0; u < 4; ++u) p[u] = (p[u] - z1) * d1;
          Bop[j] = cat(p);
          kofs[j] = gg * 64 + qh * 16 + s * 8;
        }
      } else {
        const unsigned dd[4] = {v.x, v.y, v.z, v.w};
        const _Float16 dl = __builtin_bit_cast(_Float16, (unsigned short)dmw);
        const _Float16 zz = __builtin_bit_cast(_Float16, (unsigned short)zmw);
        const f16x2 z1 = {zz, zz}, d1 = {dl, dl};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f16x2 p[4];
          unpack8_natural(dd[j], mk, p);
#pragma unroll
          for (int u = 0; u < 4; ++u) p[u] = (p[u] - z1) * d1;
          Bop[j] = cat(p);
          kofs[j] = h * 32 + j * 8;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const f16x8 A = *reinterpret_cast<const f16x8*>(xt + (16 * t + nl) * kXRow + kofs[j]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bop[j], acc[t], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 16 * t + 4 * h + r;
      if (wvalid && m < batch) store_y<OUT>(y, m * N + n, acc[t][r]);
    }
}

// Rows per wave of the VALU GEMV: batch 1 as many as keep >= 256 blocks (one per compute
// unit); batch 2 at most 4 (measured: twice the VALU work per row wants more waves).
// Rows per wave of the streaming GEMV: 8 at batch 1 when that leaves >= 256 blocks, unless the
// last round of 256 such blocks would be at most 3/8 full; then 4 rows (blocks of half the work
// even out the compute units' shares: 11008 x 4096 took 6.66 us against 7.20 with 8 rows, while
// 8192 x 8192 and 14336 x 4096, whose last rounds are whole or 3/4 full, were 5-14 % slower
// with 4).
inline int valu_rows_per_wave(int64_t N, int B) {
  if (B == 1 && N % (8 * kVWaves) == 0 && N / (8 * kVWaves) >= 256) {
    const int64_t last = (N / (8 * kVWaves)) % 256;  // blocks in the last round of the 8-row grid
    if (!(last > 0 && last <= 96)) return 8;
  }
  if (N / (4 * kVWaves) >= 256) return 4;  // N % 16 == 0
  return 2;
}

template <int B, int JMAX>
hipError_t gemv_valu_j(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gs,
                       const __half* x, void* y, int y_dtype, hipStream_t st) {
  const size_t lds = (size_t)valu_lds_bytes(B, K);
  const int gl = gs == 64 ? 6 : 7;
  const int R = valu_rows_per_wave(N, B);
  const dim3 grid((unsigned)(N / (R * kVWaves))), block(64 * kVWaves);
  if (R == 8)
    hipLaunchKernelGGL((k_gemv_valu<B, JMAX, 8>), grid, block, lds, st, packed, delta, zero, N, K, gl, y_dtype, x, y);
  else if (R == 4)
    hipLaunchKernelGGL((k_gemv_valu<B, JMAX, 4>), grid, block, lds, st, packed, delta, zero, N, K, gl, y_dtype, x, y);
  else
    hipLaunchKernelGGL((k_gemv_valu<B, JMAX, 2>), grid, block, lds, st, packed, delta, zero, N, K, gl, y_dtype, x, y);
  return hipGetLastError();
}

template <int B>
hipError_t gemv_valu(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gs,
                     const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int64_t per_lane = (K / 32 + 63) / 64;  // chunks per lane
  switch (per_lane) {
    case 1: return gemv_valu_j<B, 1>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
    case 2: return gemv_valu_j<B, 2>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
    case 3: return gemv_valu_j<B, 3>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
    case 4: return gemv_valu_j<B, 4>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
    case 5:
    case 6: return gemv_valu_j<B, 6>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
    default: return gemv_valu_j<B, 8>(packed, delta, zero, N, K, gs, x, y, y_dtype, st);
  }
}

// Batch 1-2 with rows of at most 16384 codes run on the vector ALUs.
inline bool gemv_uses_valu(int64_t K, int64_t batch) { return batch <= 2 && K <= 64 * 32 * 8; }

// Strips per block of the batched MFMA GEMV: two when that still leaves >= 256 blocks, unless
// the two-strip grid's last round of 256 blocks would be at most 3/8 full.  Then one-strip
// blocks (half the work each) even out the compute units' shares, which outweighs the x staging
// they repeat: at 11008 x 4096 (344 two-strip blocks) batch 3-6 took 8.9-10.7 us against
// 9.8-11.1 with two strips, batch 8 the same; where the last round is fuller or whole
// (14336 x 4096: 448 blocks; 28672 x 8192: 896; 8192 x 8192: 256) two strips were 2-19 % faster.
inline int mf_strips_per_block(int64_t N) {
  if (N % 32 != 0 || N / 32 < 256) return 1;
  const int64_t last = (N / 32) % 256;  // blocks in the last round of a two-strip grid
  return (last > 0 && last <= 96) ? 1 : 2;
}

template <int B, int GS, int SPB, int NSEG, int W>
void gemv_mf_launch(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                    const __half* x, void* y, int y_dtype, hipStream_t st) {
  hipLaunchKernelGGL((k_gemv_mf<B, GS, SPB, NSEG, W>), dim3((unsigned)(N / (16 * SPB))), dim3(64 * W),
                     mf_lds_bytes(B, GS, SPB, W), st, packed, delta, zero, N, K, x, y, y_dtype);
}

// Rows of up to 8192 codes: 8 waves, up to 8 segments of 1024 codes as a compile-time count
// (measured at batch 8 against 16 waves and 2048-code segments: 11008 x 4096 11.2 against 13.1 us,
// 14336 x 4096 11.6 against 13.6, 28672 x 8192 37.1 against 43.3, 8192 x 8192 12.6 against 12.7;
// the shorter segments double the pipeline's stages on short rows, and 8-wave blocks of half the
// LDS).  Longer rows (and batch 1-2, which come here only for rows past 16384 codes): 16 waves,
// 2048-code segments in a run-time loop (at 4096 x 14336 the 8-wave loop measured 15.8 against
// 14.4 us).
template <int B, int GS, int SPB>
void gemv_mf_seg(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                 const __half* x, void* y, int y_dtype, hipStream_t st) {
  if constexpr (B >= 3) {
    switch ((K + MfGeom<8>::ks - 1) / MfGeom<8>::ks) {
      case 1: return gemv_mf_launch<B, GS, SPB, 1, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 2: return gemv_mf_launch<B, GS, SPB, 2, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 3: return gemv_mf_launch<B, GS, SPB, 3, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 4: return gemv_mf_launch<B, GS, SPB, 4, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 5: return gemv_mf_launch<B, GS, SPB, 5, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 6: return gemv_mf_launch<B, GS, SPB, 6, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 7: return gemv_mf_launch<B, GS, SPB, 7, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      case 8: return gemv_mf_launch<B, GS, SPB, 8, 8>(packed, delta, zero, N, K, x, y, y_dtype, st);
      default: break;
    }
  }
  gemv_mf_launch<B, GS, SPB, 0, 16>(packed, delta, zero, N, K, x, y, y_dtype, st);
}

template <int B, int GS>
hipError_t gemv_mf(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                   const __half* x, void* y, int y_dtype, hipStream_t st) {
  if (mf_strips_per_block(N) == 2)
    gemv_mf_seg<B, GS, 2>(packed, delta, zero, N, K, x, y, y_dtype, st);
  else
    gemv_mf_seg<B, GS, 1>(packed, delta, zero, N, K, x, y, y_dtype, st);
  return hipGetLastError();
}

template <int GS>
hipError_t gemv_gs(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                   const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  const bool valu = gemv_uses_valu(K, batch);
  switch (batch) {
    case 1:
      return valu ? gemv_valu<1>(packed, delta, zero, N, K, GS, x, y, y_dtype, st)
                  : gemv_mf<1, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 2:
      return valu ? gemv_valu<2>(packed, delta, zero, N, K, GS, x, y, y_dtype, st)
                  : gemv_mf<2, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 3: return gemv_mf<3, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 4: return gemv_mf<4, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 5: return gemv_mf<5, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 6: return gemv_mf<6, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 7: return gemv_mf<7, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 8: return gemv_mf<8, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemv_lds_bytes(int64_t K, int gs, int64_t batch) {
  if (gemv_uses_valu(K, batch)) return (size_t)valu_lds_bytes((int)batch, K);
  if (batch < 1 || batch > 8) return 0;
  return (size_t)mf_lds_bytes((int)batch, gs, 2, 16);  // the two-strip 16-wave layout is the largest
}

hipError_t launch_gemv(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gs,
                       const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  return gs == 64 ? gemv_gs<64>(packed, delta, zero, N, K, x, batch, y, y_dtype, st)
                  : gemv_gs<128>(packed, delta, zero, N, K, x, batch, y, y_dtype, st);
}

hipError_t launch_gemm(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gs,
                       const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  const dim3 grid((unsigned)((batch + kGemmM - 1) / kGemmM), (unsigned)((N + 63) / 64));
  if (gs == 64) {
    if (y_dtype == HQQ_OUT_F16)
      hipLaunchKernelGGL((k_gemm<64, HQQ_OUT_F16>), grid, dim3(256), 0, st, packed, delta, zero, N, K, x, batch, y);
    else
      hipLaunchKernelGGL((k_gemm<64, HQQ_OUT_F32>), grid, dim3(256), 0, st, packed, delta, zero, N, K, x, batch, y);
  } else {
    if (y_dtype == HQQ_OUT_F16)
      hipLaunchKernelGGL((k_gemm<128, HQQ_OUT_F16>), grid, dim3(256), 0, st, packed, delta, zero, N, K, x, batch, y);
    else
      hipLaunchKernelGGL((k_gemm<128, HQQ_OUT_F32>), grid, dim3(256), 0, st, packed, delta, zero, N, K, x, batch, y);
  }
  return hipGetLastError();
}

}  // namespace hqq
