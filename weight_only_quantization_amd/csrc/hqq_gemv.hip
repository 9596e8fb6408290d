// Fused dequantise + product, 4-bit weights, fp16 activations, fp32 accumulation (page
// "HQQ 算法解读", section "从压缩文件到一次前向": unpack, (q - zero) * scale, x @ W_hat^T).
//
// Both kernels run on the MFMA unit (v_mfma_f32_16x16x32_f16): the weight tile is the B
// operand (16 output rows n per tile, n = lane % 16), the activations are the A operand
// (16 batch rows m per tile, m = lane % 16), and lane (h = lane / 16, r) of the result holds
// y[m = 4h + r][n].
//
// Weight streaming: lane (h, n) loads 16 bytes (32 codes) of row n per 128-code chunk, so a
// wave reads 16 rows x 64 contiguous bytes per load instruction.  One v_permlane32_swap per
// dword pair regroups the chunk so that the four lane groups hold the four 16-code quarters of
// one 64-code group (lane group h holds quarter pi(h), pi = [0, 2, 1, 3]): every MFMA then sums
// codes of a single group, which lets the group's delta and zero be applied once per group.
//
// Code unpack ("magic" fp16): for a dword of eight 4-bit codes c0..c7,
//   (d & 0x000F000F) | 0x64006400 = fp16 (1024 + c0, 1024 + c4),
//   (d & 0x00F000F0) | 0x64006400 = fp16 (1024 + 16 c1, 1024 + 16 c5), and the same on d >> 8;
// one packed fp16 add of -1024 leaves exact small integers.  The operand order within the
// lane's eight k slots is therefore [0, 4, 1, 5, 2, 6, 3, 7] with a factor 16 on the odd codes;
// the activations are staged in the same order (and, in the GEMV, with 1/16 on the odd codes).
//
// GEMV (batch <= 8): q stays exact; the MFMA forms P = sum_k x_k q_k per group and the group's
// metadata is applied on the fp32 partial: acc += delta * (P - z * sum_k x_k).
// GEMM (batch > 8): the tile is dequantised to fp16 W_hat = (q - z) * delta first (the plain
// "dequantise then matmul" of the page, with fp32 accumulation).

#include "hqq_gemv_common.h"

namespace hqq {
namespace {

// ------------------------------------------------------------------------------------------
// GEMV, batch B <= 8.  Block = 8 waves on SPB 16-row strips; wave w takes the 128-code chunks
// c = w, w + 8, ... of each K segment, for every strip of the block.  Per segment the
// activations are staged in LDS in the operand order (x, with 1/16 on odd codes) together with
// the per-group sums of x (staged once for all SPB strips), and so are the packed codes: wave w
// loads whole row segments (rows w, w + 8, ...: one 1 KB run, one page, per load instruction;
// the MFMA operand layout would put 16 rows, 16 pages, into every instruction) and each lane
// then reads its 16-byte operand pieces from LDS.  The next segment's loads are in flight
// while the current one is multiplied.  The eight waves' partial results are added in a fixed
// order at the end.
// ------------------------------------------------------------------------------------------
template <int B>
struct GemvCfg {
  static constexpr int CPW = (B <= 2) ? 8 : (B <= 4 ? 4 : 2);  // chunks per wave per segment
  static constexpr int KS = 128 * 8 * CPW;                       // K per segment
};

template <int B, int GS, int OUT, int SPB>
__global__ void __launch_bounds__(512) k_gemv(const uint8_t* __restrict__ packed, const __half* __restrict__ delta,
                                              const __half* __restrict__ zero, int64_t N, int64_t K,
                                              const __half* __restrict__ x, void* __restrict__ y) {
  constexpr int CPW = GemvCfg<B>::CPW, KS = GemvCfg<B>::KS;
  constexpr int GPS = KS / GS;  // groups per segment
  constexpr int KSP = KS + 8;   // LDS row stride of x: padded so that rows fall in different banks
  constexpr int WRB = KS / 2 + 16;  // LDS row stride of the packed codes (bytes; 16 rows, distinct banks)
  constexpr int RPW = SPB * 2;      // weight rows each wave loads per segment
  constexpr int PPL = KS / 32 / 64; // 16-byte pieces of a row segment per lane
  extern __shared__ float lds[];
  float* sx = lds;                                                     // [B][GPS]
  float* red = sx + B * GPS;                                           // [SPB][8][B][16]
  _Float16* xs = reinterpret_cast<_Float16*>(red + SPB * 8 * B * 16);  // [B][KSP]
  uint8_t* wl = reinterpret_cast<uint8_t*>(xs + B * KSP);              // [16 SPB][WRB] packed codes

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 4, nl = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * SPB;
  const int64_t gpr = K / GS;  // groups per row
  const int qh = quarter_of(h);
  // A-operand row of this lane: batch rows >= B read row 0; they only feed output rows >= B,
  // which are never stored.
  const int arow = nl < B ? nl : 0;

  f32x4 acc[SPB];
#pragma unroll
  for (int sp = 0; sp < SPB; ++sp) acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t nchunks = K / 128;
  constexpr int XR = (B * (KS / 8) + 511) / 512;  // 8-element blocks of x staged per thread
  // Loads of one segment: this thread's blocks of x (small, cache-resident) first, so that
  // staging them does not wait for the weight stream, then the wave's weight chunks.  All loads
  // are unconditional (clamped indexes): a load under a branch makes the compiler wait for it
  // before the branch joins; blocks and chunks past the end are never staged or never used.
  uint4 xr[XR];
  uint4 wr[RPW][PPL];  // this wave's row segments of packed codes (PPL 16-byte pieces per lane and row)
  unsigned dm[SPB][CPW], zm[SPB][CPW], dmn[SPB][CPW], zmn[SPB][CPW];
  auto load_segment = [&](int64_t kb0, unsigned (&d)[SPB][CPW], unsigned (&z)[SPB][CPW]) {
    const int nbs = (int)(((K - kb0 < KS) ? (K - kb0) : KS) / 8);
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = tid + 512 * j;
      const int m = min(idx / (KS / 8), B - 1), kb = min(idx % (KS / 8), nbs - 1);
      xr[j] = *reinterpret_cast<const uint4*>(x + m * K + kb0 + 8 * kb);
    }
#pragma unroll
    for (int sp = 0; sp < SPB; ++sp) {
      const int64_t n = n0 + 16 * sp + nl;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int64_t c = min(kb0 / 128 + wave + 8 * i, nchunks - 1);
        if constexpr (GS == 64) {
          d[sp][i] = *reinterpret_cast<const unsigned*>(delta + n * gpr + 2 * c);
          z[sp][i] = *reinterpret_cast<const unsigned*>(zero + n * gpr + 2 * c);
        } else {
          d[sp][i] = __half_as_ushort(delta[n * gpr + c]);
          z[sp][i] = __half_as_ushort(zero[n * gpr + c]);
        }
      }
    }
    {
      const int pieces = (int)(((K - kb0 < KS) ? (K - kb0) : KS) / 32);  // 16-byte pieces of the segment's rows
#pragma unroll
      for (int j = 0; j < RPW; ++j)
#pragma unroll
        for (int q = 0; q < PPL; ++q)
          wr[j][q] = ld_stream16(packed + (n0 + wave + 8 * j) * (K / 2) + kb0 / 2 + 16 * min(lane + 64 * q, pieces - 1));
    }
  };
  load_segment(0, dm, zm);
  for (int64_t kbase = 0; kbase < K; kbase += KS) {
    const int64_t cbase = kbase / 128;
    // 1. stage x in operand order (1/16 on the odd codes) with the per-group sums of x
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = tid + 512 * j;
      if (idx < B * (KS / 8)) {  // uniform per 256-lane run: segments of GS/8 lanes stay whole
        const int m = idx / (KS / 8), kb = idx % (KS / 8);
        const uint4 raw = xr[j];
        const unsigned r4[4] = {raw.x, raw.y, raw.z, raw.w};
        float part = block_sum8(r4);
        uint4 o = perm_slots(raw);
        o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        *reinterpret_cast<uint4*>(xs + m * KSP + 8 * kb) = o;
        part = seg_sum_f<GS / 8>(part);
        if ((kb % (GS / 8)) == 0) sx[m * GPS + kb / (GS / 8)] = part;
      }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int q = 0; q < PPL; ++q) *reinterpret_cast<uint4*>(wl + (wave + 8 * j) * WRB + 16 * (lane + 64 * q)) = wr[j][q];
    // this segment's steps and zeros, requested with its codes (no earlier wait than the codes')
    if (kbase > 0) {
#pragma unroll
      for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
          dm[sp][i] = dmn[sp][i];
          zm[sp][i] = zmn[sp][i];
        }
    }
    lds_barrier();  // LDS hand-over
    // 2. the next segment's loads go out before this one is multiplied
    const bool more = kbase + KS < K;
    if (more) load_segment(kbase + KS, dmn, zmn);
    uint4 v[SPB][CPW];
#pragma unroll
    for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int cl = min(wave + 8 * i, KS / 128 - 1);  // chunk within the segment (unused when past the end)
        v[sp][i] = *reinterpret_cast<const uint4*>(wl + (16 * sp + nl) * WRB + cl * 64 + h * 16);
      }

#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int64_t c = cbase + wave + 8 * i;
      if (c >= nchunks) break;
      const int cl = (int)(c - cbase);  // chunk within the segment
      if constexpr (GS == 64) {
        const int kl = cl * 128 + qh * 16;
        const f16x8 a00 = *reinterpret_cast<const f16x8*>(xs + arow * KSP + kl);
        const f16x8 a01 = *reinterpret_cast<const f16x8*>(xs + arow * KSP + kl + 8);
        const f16x8 a10 = *reinterpret_cast<const f16x8*>(xs + arow * KSP + kl + 64);
        const f16x8 a11 = *reinterpret_cast<const f16x8*>(xs + arow * KSP + kl + 72);
        float sx0[4], sx1[4];
#pragma unroll
        for (int r = 0; r < (B < 4 ? B : 4); ++r) {
          const int m = 4 * h + r;
          sx0[r] = (m < B) ? sx[m * GPS + cl * 2] : 0.f;
          sx1[r] = (m < B) ? sx[m * GPS + cl * 2 + 1] : 0.f;
        }
#pragma unroll
        for (int sp = 0; sp < SPB; ++sp) {
          // regroup: lane group h then holds quarter pi(h) of both 64-code groups of the chunk
          const auto s0 = __builtin_amdgcn_permlane32_swap(v[sp][i].x, v[sp][i].z, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(v[sp][i].y, v[sp][i].w, false, false);
          const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
          // the two groups' products interleaved (no back-to-back dependent MFMA)
          f32x4 P0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a00, unpack8_sub(s0[0]), zero4, 0, 0, 0);
          f32x4 P1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a10, unpack8_sub(s0[1]), zero4, 0, 0, 0);
          P0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a01, unpack8_sub(s1[0]), P0, 0, 0, 0);
          P1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a11, unpack8_sub(s1[1]), P1, 0, 0, 0);
          // P = 2^-24 sum x q: scale the step up and the zero down by 2^24 (exact)
          const float dl0 = __half2float(__ushort_as_half((unsigned short)dm[sp][i])) * kSubScale;
          const float dl1 = __half2float(__ushort_as_half((unsigned short)(dm[sp][i] >> 16))) * kSubScale;
          const float zz0 = __half2float(__ushort_as_half((unsigned short)zm[sp][i])) * kSubScaleInv;
          const float zz1 = __half2float(__ushort_as_half((unsigned short)(zm[sp][i] >> 16))) * kSubScaleInv;
#pragma unroll
          for (int r = 0; r < (B < 4 ? B : 4); ++r) {
            acc[sp][r] = fmaf(dl0, fmaf(-zz0, sx0[r], P0[r]), acc[sp][r]);
            acc[sp][r] = fmaf(dl1, fmaf(-zz1, sx1[r], P1[r]), acc[sp][r]);
          }
        }
      } else {  // GS == 128: the 128-code chunk is one group; lane group h holds codes 32h..32h+31
        f16x8 A[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) A[t] = *reinterpret_cast<const f16x8*>(xs + arow * KSP + cl * 128 + h * 32 + t * 8);
        float sxv[4];
#pragma unroll
        for (int r = 0; r < (B < 4 ? B : 4); ++r) {
          const int m = 4 * h + r;
          sxv[r] = (m < B) ? sx[m * GPS + cl] : 0.f;
        }
#pragma unroll
        for (int sp = 0; sp < SPB; ++sp) {
          const unsigned dd[4] = {v[sp][i].x, v[sp][i].y, v[sp][i].z, v[sp][i].w};
          f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], unpack8_sub(dd[t]), P, 0, 0, 0);
          const float dl = __half2float(__ushort_as_half((unsigned short)dm[sp][i])) * kSubScale;
          const float zz = __half2float(__ushort_as_half((unsigned short)zm[sp][i])) * kSubScaleInv;
#pragma unroll
          for (int r = 0; r < (B < 4 ? B : 4); ++r) acc[sp][r] = fmaf(dl, fmaf(-zz, sxv[r], P[r]), acc[sp][r]);
        }
      }
    }
    lds_barrier();  // LDS hand-over; the next segment's loads stay in flight
  }
#pragma unroll
  for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
    for (int r = 0; r < (B < 4 ? B : 4); ++r) {
      const int m = 4 * h + r;
      if (m < B) red[((sp * 8 + wave) * B + m) * 16 + nl] = acc[sp][r];
    }
  __syncthreads();
  if (tid < SPB * B * 16) {
    const int sp = tid / (B * 16), m = (tid / 16) % B, col = tid % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[((sp * 8 + w) * B + m) * 16 + col];
    store_y<OUT>(y, (int64_t)m * N + n0 + 16 * sp + col, sum);
  }
}

// ------------------------------------------------------------------------------------------
// GEMV on the vector ALUs, batch B <= 2.  Each wave streams whole rows: lane l takes the
// 32-code chunks c = l + 64 j of a row, so one load instruction reads 1 KB of one row.  Per
// chunk the lane forms P = sum x_k q_k with v_dot2_f32_f16 on exact codes and applies the
// group's step and zero on the fp32 partial, acc += delta * (P - z * sum_k x_k); row results
// are reduced over the wave's lanes with a fixed tree.
//
// Pipelining: wave gw of the grid takes exactly R rows, n = gw + k * (N / R), so at any time
// the waves of the chip stream one contiguous band of rows.  D rows are in flight per wave:
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
  const int64_t TW = N / R;                    // waves in the grid
  const int64_t gw = (int64_t)blockIdx.x * W + wave;

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
inline int valu_rows_per_wave(int64_t N, int B) {
  if (B == 1 && N % (8 * kVWaves) == 0 && N / (8 * kVWaves) >= 256) return 8;
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

template <int B>
size_t gemv_lds_b(int gs, int spb) {
  constexpr int KS = GemvCfg<B>::KS;
  return (size_t)B * (KS / gs) * 4 + (size_t)spb * 8 * B * 16 * 4 + (size_t)B * (KS + 8) * 2 +
         (size_t)16 * spb * (KS / 2 + 16);
}

// Strips per block of the batched GEMV: two when that still leaves >= 256 blocks.
inline int gemv_strips_per_block(int64_t N, int64_t batch) {
  return (batch >= 3 && N % 32 == 0 && N / 32 >= 256) ? 2 : 1;  // batch <= 2 holds 8 chunks per strip
}

template <int B, int GS>
hipError_t gemv_b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                  const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int spb = gemv_strips_per_block(N, B);
  const size_t lds = gemv_lds_b<B>(GS, spb);
  const dim3 grid((unsigned)(N / (16 * spb)));
  if constexpr (B >= 3) {
    if (spb == 2) {
      if (y_dtype == HQQ_OUT_F16)
        hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F16, 2>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
      else
        hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F32, 2>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
      return hipGetLastError();
    }
  }
  {
    if (y_dtype == HQQ_OUT_F16)
      hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F16, 1>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
    else
      hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F32, 1>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
  }
  return hipGetLastError();
}

// Batch 1-2 with rows of at most 16384 codes run on the vector ALUs.
inline bool gemv_uses_valu(int64_t K, int64_t batch) { return batch <= 2 && K <= 64 * 32 * 8; }

template <int GS>
hipError_t gemv_gs(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                   const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  const bool valu = gemv_uses_valu(K, batch);
  switch (batch) {
    case 1:
      return valu ? gemv_valu<1>(packed, delta, zero, N, K, GS, x, y, y_dtype, st)
                  : gemv_b<1, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 2:
      return valu ? gemv_valu<2>(packed, delta, zero, N, K, GS, x, y, y_dtype, st)
                  : gemv_b<2, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 3: return gemv_b<3, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 4: return gemv_b<4, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 5: return gemv_b<5, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 6: return gemv_b<6, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 7: return gemv_b<7, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 8: return gemv_b<8, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemv_lds_bytes(int64_t K, int gs, int64_t batch) {
  if (gemv_uses_valu(K, batch)) return (size_t)valu_lds_bytes((int)batch, K);
  switch (batch) {  // the larger of the one- and two-strip layouts
    case 1: return gemv_lds_b<1>(gs, 2);
    case 2: return gemv_lds_b<2>(gs, 2);
    case 3: return gemv_lds_b<3>(gs, 2);
    case 4: return gemv_lds_b<4>(gs, 2);
    case 5: return gemv_lds_b<5>(gs, 2);
    case 6: return gemv_lds_b<6>(gs, 2);
    case 7: return gemv_lds_b<7>(gs, 2);
    case 8: return gemv_lds_b<8>(gs, 2);
    default: return 0;
  }
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
