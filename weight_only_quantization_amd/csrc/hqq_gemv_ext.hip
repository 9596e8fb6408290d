// Fused dequantise + product for the other stored formats (page "HQQ 算法解读", sections
// "从压缩文件到一次前向": unpack, (q - zero) * scale, x @ W_hat^T; "`axis` 不是一个无关紧要的开关"
// for the axis-0 groups; "为什么一定要分组" for the 2-bit container):
//   * 4-bit codes with axis-0 groups (a group is a column of reshape([g, -1]): weight row n
//     uses metadata row r0 = n mod (N/g), one step and zero per column k);
//   * 2-bit codes with axis-1 groups of 16 (four codes per byte, one group per 32-bit word).
// Both run on the vector ALUs with v_dot2_f32_f16 on exact codes (fp16 subnormals, as in the
// 4-bit kernels) and stream whole weight rows, 1 KB per load instruction.

#include <type_traits>

#include "hqq_gemv_common.h"

namespace hqq {
namespace {

// ------------------------------------------------------------------------------------------
// Axis 0, 4-bit.  For metadata row r0 the product is
//   y[b, n] = sum_k a[b, k] q[n, k] - sum_k a[b, k] z[r0, k],   a[b, k] = x[b, k] delta[r0, k],
// so a block takes one r0 (and a share of its g weight rows n = r0 + (N/g) i): it forms a in
// fp16 (the product of two fp16 values, rounded once), staged in the unpack slot order with
// 1/16 on the odd codes, and the zero term from the same staged values (so both terms use the
// same weights); every weight row is then one fp16-dot-product pass over exact codes.
// ------------------------------------------------------------------------------------------
constexpr int kAx0Waves = 4;

template <int B, int JMAX, int RPW, int D>
__global__ void __launch_bounds__(64 * kAx0Waves) k_gemv_ax0(const uint8_t* __restrict__ packed,
                                                            const __half* __restrict__ delta,
                                                            const __half* __restrict__ zero, int64_t N, int64_t K,
                                                            int g, int subsets, int out_dtype,
                                                            const __half* __restrict__ x, void* __restrict__ y) {
  static_assert(D >= 1 && D <= RPW, "rows in flight must be within the wave's rows");  // D: rows in flight
  constexpr bool XREG = B * JMAX <= 4;      // a chunks held in registers
  constexpr int NT = 64 * kAx0Waves;
  extern __shared__ float lds[];
  const int nch = (int)(K / 32);            // 32-code chunks per row
  float* red = lds;                         // [waves][B] partial zero terms
  uint4* as = reinterpret_cast<uint4*>(red + 4 * B);  // [B][4][nch] 16-byte blocks of a
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t R0 = N / g;
  const int64_t r0 = blockIdx.x / subsets;
  const int sub = blockIdx.x % subsets;
  const __half* drow = delta + r0 * K;
  const __half* zrow = zero + r0 * K;
  // rows of this wave: i = sub * 4 * RPW + wave * RPW + t, n = r0 + R0 * i
  const int64_t i0 = (int64_t)sub * kAx0Waves * RPW + wave * RPW;

  // 1. x, delta and zero blocks of this thread (a block past the end re-reads the last one)
  constexpr int XR = (B * 64 * JMAX * 4 + NT - 1) / NT;
  const int nxb = B * nch * 4;
  uint4 xr[XR], dr[XR], zr[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = min(tid + NT * i, nxb - 1);
    const int kb = idx % (nch * 4);
    xr[i] = *reinterpret_cast<const uint4*>(x + 8 * idx);  // x is [B][K] contiguous
    dr[i] = *reinterpret_cast<const uint4*>(drow + 8 * kb);
    zr[i] = *reinterpret_cast<const uint4*>(zrow + 8 * kb);
  }
  __builtin_amdgcn_sched_barrier(0);  // these loads go out ahead of the weight stream

  // 2. the first D rows of this wave, in flight
  uint4 wv[D][JMAX];
  auto issue = [&](int s, int64_t i) {
    const uint8_t* wrow = packed + (r0 + R0 * i) * (K / 2);
#pragma unroll
    for (int j = 0; j < JMAX; ++j) wv[s][j] = ld_stream16(wrow + 16 * min(lane + 64 * j, nch - 1));
  };
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, i0 + s);

  // 3. stage a = x * delta (fp16) in the unpack order, 1/16 on the odd codes, and the zero term
  float zpart[B];
#pragma unroll
  for (int b = 0; b < B; ++b) zpart[b] = 0.f;
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx_raw = tid + NT * i;
    const int idx = min(idx_raw, nxb - 1);
    const int m = idx / (nch * 4), rem = idx % (nch * 4), c = rem / 4, t = rem % 4;
    const unsigned xu[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
    const unsigned du[4] = {dr[i].x, dr[i].y, dr[i].z, dr[i].w};
    const unsigned zu[4] = {zr[i].x, zr[i].y, zr[i].z, zr[i].w};
    unsigned au[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x2 xv = as_h2(xu[q]), dv = as_h2(du[q]);
      const f16x2 av = {(_Float16)((float)xv[0] * (float)dv[0]), (_Float16)((float)xv[1] * (float)dv[1])};
      au[q] = as_u(av);
    }
    uint4 o = perm_slots(make_uint4(au[0], au[1], au[2], au[3]));
    o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
    o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
    as[(m * 4 + t) * nch + c] = o;
    // zero term from the staged values: slot order [k0, k4, k1, k5, k2, k6, k3, k7], odd x 16
    const uint4 zp = perm_slots(make_uint4(zu[0], zu[1], zu[2], zu[3]));
    const unsigned ou[4] = {o.x, o.y, o.z, o.w}, zq[4] = {zp.x, zp.y, zp.z, zp.w};
    float zt = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sc = (q & 1) ? 16.f : 1.f;
      zt = fmaf((float)as_h2(ou[q])[0] * sc, (float)as_h2(zq[q])[0], zt);
      zt = fmaf((float)as_h2(ou[q])[1] * sc, (float)as_h2(zq[q])[1], zt);
    }
    if (idx_raw < nxb) {
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (m == b) zpart[b] += zt;
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = wave_sum(zpart[b]);
    if (lane == 0) red[wave * B + b] = v;
  }
  lds_barrier();  // LDS hand-over; the weight loads stay in flight
  float zb[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kAx0Waves; ++w) v += red[w * B + b];
    zb[b] = v;
  }
  f16x2 aq[XREG ? B : 1][XREG ? JMAX : 1][16];
  if constexpr (XREG) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < JMAX; ++j) {
        const int c = min(lane + 64 * j, nch - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 v = as[(b * 4 + t) * nch + c];
          aq[b][j][4 * t + 0] = as_h2(v.x);
          aq[b][j][4 * t + 1] = as_h2(v.y);
          aq[b][j][4 * t + 2] = as_h2(v.z);
          aq[b][j][4 * t + 3] = as_h2(v.w);
        }
      }
  }

  // 4. rows: multiply row t, then request row t + D into the freed slot
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int s = t % D;
    const int64_t n = r0 + R0 * (i0 + t);
    float P[B];
#pragma unroll
    for (int b = 0; b < B; ++b) P[b] = 0.f;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      const bool valid = lane + 64 * j < nch;
      const unsigned dw[4] = {wv[s][j].x, wv[s][j].y, wv[s][j].z, wv[s][j].w};
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float p = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 u = __builtin_bit_cast(u32x4, unpack8_sub(dw[q]));
          if constexpr (XREG) {
#pragma unroll
            for (int e = 0; e < 4; ++e) p = __builtin_amdgcn_fdot2(aq[b][j][4 * q + e], as_h2(u[e]), p, false);
          } else {
            const uint4 av = as[(b * 4 + q) * nch + c];
            const unsigned au[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) p = __builtin_amdgcn_fdot2(as_h2(au[e]), as_h2(u[e]), p, false);
          }
        }
        P[b] += valid ? p : 0.f;
      }
    }
    if (t + D < RPW) issue(s, i0 + t + D);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum(P[b]) * kSubScale - zb[b];
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
// Axis 0, 4-bit, batch 3..8, on the MFMA unit.  The same factorisation as k_gemv_ax0 (a block
// takes RB = 16 SPB of the g weight rows of one metadata row r0, a = x delta[r0] in fp16, the
// zero term sum_k a z[r0, k] from the same staged values), with the segment pipeline of the
// 4-bit batch 3-8 kernel: W waves (8 for rows of up to 8192 codes, 16 beyond), K in segments
// of 128 W codes, wave w always takes the 128-code chunk w of a segment; per segment the block
// stages a (unpack slot order, 1/16 on the odd codes) and the packed rows (1 KB of one or two
// rows per load instruction) in LDS, double buffered, the loads two segments ahead in
// registers, one LDS-only barrier per segment.
// The codes stay exact (fp16 subnormals into v_mfma_f32_16x16x32_f16) and there is no
// per-group step inside a row, so each wave's MFMAs chain over the whole row:
//   y[b, n] = 2^24 sum_w P_w[b, n] - sum_k a[b, k] z[r0, k],
// the W waves' sums added in wave order, the zero term in a fixed tree (deterministic).
// ------------------------------------------------------------------------------------------
// LDS bytes of one stage of W waves (a, then the packed rows).
__host__ __device__ constexpr int mf0_stage_bytes(int B, int SPB, int W) {
  return B * (128 * W + 8) * 2 + 16 * SPB * (64 * W + 16);
}

template <int B, int SPB, int NSEG, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_mf0(const uint8_t* __restrict__ packed,
                                                    const __half* __restrict__ delta,
                                                    const __half* __restrict__ zero, int64_t N, int64_t K,
                                                    int g, int subsets, int xcd_map, int out_dtype,
                                                    const __half* __restrict__ x, void* __restrict__ y) {
  static_assert(B >= 1 && B <= 8 && (SPB == 1 || SPB == 2) && (W == 8 || W == 16), "shape");
  constexpr int kM0Waves = W;
  constexpr int kM0KS = 128 * W;        // codes per segment
  constexpr int kM0KSP = kM0KS + 8;     // LDS row stride of a (halves)
  constexpr int kM0WRB = kM0KS / 2 + 16;  // LDS row stride of the packed codes (bytes)
  constexpr int kPieces = kM0KS / 32;   // 16-byte pieces of one row's segment of codes
  constexpr int kRowsPerWave = 16 / W;  // rows of a strip each wave loads per segment
  constexpr int NT = 64 * kM0Waves, RB = 16 * SPB;
  constexpr int XB = B * (kM0KS / 8);      // 16-byte blocks of x (and of a) per segment
  constexpr int XR = (XB + NT - 1) / NT;   // of them per thread
  constexpr int STAGE = mf0_stage_bytes(B, SPB, W);
  extern __shared__ __align__(16) uint8_t lds_raw[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 4, nl = lane & 15;
  const int arow = nl < B ? nl : 0;  // A rows >= B only feed outputs that are never stored
  // Block b runs on XCD b mod 8 (round-robin dispatch).  With xcd_map (N / g a multiple of 8) the
  // `subsets` blocks of one metadata row share an XCD, so its steps and zeros come from that L2.
  const int64_t R0 = N / g;
  int64_t r0, sub;
  if (xcd_map) {
    const int64_t xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    r0 = 8 * (q / subsets) + xcd;
    sub = q % subsets;
  } else {
    r0 = blockIdx.x / subsets;
    sub = blockIdx.x % subsets;
  }
  const int64_t i0 = sub * RB;  // rows n = r0 + R0 (i0 + row)
  const __half* drow = delta + r0 * K;
  const __half* zrow = zero + r0 * K;
  const int64_t nchunks = K / 128;
  const int nseg = NSEG > 0 ? NSEG : (int)((K + kM0KS - 1) / kM0KS);

  auto as_of = [&](int buf) { return reinterpret_cast<_Float16*>(lds_raw + buf * STAGE); };
  auto wl_of = [&](int buf) { return lds_raw + buf * STAGE + B * kM0KSP * 2; };

  struct Regs {
    uint4 xr[XR], dr[XR], zr[XR];
    uint4 wr[SPB];
  };
  auto load_seg = [&](int sg, Regs& r) {
    const int64_t kb0 = (int64_t)sg * kM0KS;
    const int valid = (int)((K - kb0 < kM0KS) ? (K - kb0) : kM0KS);  // a multiple of 128
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = min(tid + NT * j, XB - 1);
      const int m = idx / (kM0KS / 8), kb = min(idx % (kM0KS / 8), valid / 8 - 1);
      r.xr[j] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + kb0 + 8 * kb);
      r.dr[j] = *reinterpret_cast<const uint4*>(drow + kb0 + 8 * kb);
      r.zr[j] = *reinterpret_cast<const uint4*>(zrow + kb0 + 8 * kb);
    }
#pragma unroll
    for (int j = 0; j < SPB; ++j) {  // each wave takes 16 / W rows of the strip
      const int row = kRowsPerWave * wave + lane / kPieces + 16 * j;
      const int piece = min(lane % kPieces, valid / 32 - 1);
      r.wr[j] = ld_stream16(packed + (r0 + R0 * (i0 + row)) * (K / 2) + kb0 / 2 + 16 * piece);
    }
  };
  // a = x delta -> LDS stage `buf`; the zero term of the thread's blocks into zacc
  float zacc[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) zacc[j] = 0.f;
  auto stage_seg = [&](int sg, int buf, const Regs& r) {
    const int64_t kb0 = (int64_t)sg * kM0KS;
    const int valid = (int)((K - kb0 < kM0KS) ? (K - kb0) : kM0KS);
    _Float16* as = as_of(buf);
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int idx = tid + NT * j;
      if (idx < XB) {  // uniform per wave (XB is a multiple of 128 W / 8 >= 128)
        const int m = idx / (kM0KS / 8), kb = idx % (kM0KS / 8);
        const unsigned xu[4] = {r.xr[j].x, r.xr[j].y, r.xr[j].z, r.xr[j].w};
        const unsigned du[4] = {r.dr[j].x, r.dr[j].y, r.dr[j].z, r.dr[j].w};
        unsigned au[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x2 xv = as_h2(xu[q]), dv = as_h2(du[q]);
          au[q] = as_u(f16x2{(_Float16)((float)xv[0] * (float)dv[0]), (_Float16)((float)xv[1] * (float)dv[1])});
        }
        uint4 o = perm_slots(make_uint4(au[0], au[1], au[2], au[3]));
        o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        *reinterpret_cast<uint4*>(as + m * kM0KSP + 8 * kb) = o;
        // zero term from the staged values: slot order [k0, k4, k1, k5, k2, k6, k3, k7], odd x 16
        const uint4 zp = perm_slots(r.zr[j]);
        const unsigned ou[4] = {o.x, o.y, o.z, o.w}, zq[4] = {zp.x, zp.y, zp.z, zp.w};
        float zt = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = (q & 1) ? 16.f : 1.f;
          zt = fmaf((float)as_h2(ou[q])[0] * sc, (float)as_h2(zq[q])[0], zt);
          zt = fmaf((float)as_h2(ou[q])[1] * sc, (float)as_h2(zq[q])[1], zt);
        }
        if (8 * kb < valid) zacc[j] += zt;
      }
    }
    uint8_t* wl = wl_of(buf);
#pragma unroll
    for (int j = 0; j < SPB; ++j)
      *reinterpret_cast<uint4*>(wl + (kRowsPerWave * wave + lane / kPieces + 16 * j) * kM0WRB + 16 * (lane % kPieces)) =
          r.wr[j];
  };

  f32x4 acc[SPB];
#pragma unroll
  for (int sp = 0; sp < SPB; ++sp) acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
  Regs rs[2];
  load_seg(0, rs[0]);
  if (NSEG != 1) load_seg(min(1, nseg - 1), rs[1]);
  stage_seg(0, 0, rs[0]);
  if (NSEG == 0 || NSEG > 2) load_seg(min(2, nseg - 1), rs[0]);
  lds_barrier();
  // one segment: stage `cur` + 1 (requested two segments earlier) into the other stage, refill
  // that register set with `cur` + 3, multiply `cur`; one LDS-only barrier
  auto segment = [&](const int cur, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (cur + 1 < nseg) stage_seg(cur + 1, buf ^ 1, rs[buf ^ 1]);
    if (NSEG == 0 || cur + 3 < NSEG) load_seg(min(cur + 3, nseg - 1), rs[buf ^ 1]);
    const int64_t c = (int64_t)cur * kM0Waves + wave;  // this wave's chunk
    if (c < nchunks) {
      const _Float16* as = as_of(buf);
      const uint8_t* wl = wl_of(buf);
      // lane group h holds codes 32 h .. 32 h + 31 of the chunk, dword t codes 8 t .. 8 t + 7
      f16x8 A[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        A[t] = *reinterpret_cast<const f16x8*>(as + arow * kM0KSP + wave * 128 + h * 32 + t * 8);
#pragma unroll
      for (int sp = 0; sp < SPB; ++sp) {
        const uint4 v = *reinterpret_cast<const uint4*>(wl + (16 * sp + nl) * kM0WRB + wave * 64 + h * 16);
        const unsigned dd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[sp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], unpack8_sub(dd[t]), acc[sp], 0, 0, 0);
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
  // ---- the W waves' sums of each output in wave order, the zero term in a fixed tree (the
  //      wave's 64 lanes, then the W / 4 waves of a batch row); stage memory reused
  float* red = reinterpret_cast<float*>(lds_raw);  // [SPB][W waves][B][16]
  float* redz = red + SPB * kM0Waves * B * 16;      // [XR][W waves]
#pragma unroll
  for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * h + r;
      if (m < B) red[((sp * kM0Waves + wave) * B + m) * 16 + nl] = acc[sp][r];
    }
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const float v = wave_sum(zacc[j]);
    if (lane == 0) redz[j * kM0Waves + wave] = v;
  }
  lds_barrier();
  if (tid < SPB * B * 16) {
    const int sp = tid / (B * 16), m = (tid / 16) % B, col = tid % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kM0Waves; ++w) sum += red[((sp * kM0Waves + w) * B + m) * 16 + col];
    // batch row m: blocks idx = tid + NT j with idx / (16 W) = m, i.e. j = m / 4, waves
    // (W / 4) (m % 4) + 0 .. W / 4 - 1
    const float* zw = redz + (m / 4) * kM0Waves + (W / 4) * (m % 4);
    const float zb = W == 16 ? (zw[0] + zw[1]) + (zw[2] + zw[3]) : zw[0] + zw[1];
    const float v = sum * kSubScale - zb;
    const int64_t n = r0 + R0 * (i0 + 16 * sp + col);
    if (out_dtype == HQQ_OUT_F16)
      store_y<HQQ_OUT_F16>(y, (int64_t)m * N + n, v);
    else
      store_y<HQQ_OUT_F32>(y, (int64_t)m * N + n, v);
  }
}

// ------------------------------------------------------------------------------------------
// Axis 1, 2-bit, groups of 16 (one group per 32-bit word).  Lane l takes the 16-byte chunks
// c = l + 64 j of a row (64 codes, four groups).  A word d gives its 16 codes as fp16
// subnormals with one AND each pair: d & 0x00030003 = (c0, c8), d & 0x000C000C = (4c1, 4c9),
// d & 0x00300030 = (16c2, 16c10), d & 0x00C000C0 = (64c3, 64c11), and the same on d >> 8 for
// c4..c7 / c12..c15; x is staged in that pair order with 1, 1/4, 1/16, 1/64 on the four
// positions.  Per group: acc += delta * (P - z * sum_k x_k), the 2^24 folded into delta and z.
// Waves take R consecutive rows with two rows in flight, as the 4-bit kernel.
// ------------------------------------------------------------------------------------------
constexpr int k2Waves = 4;

__device__ __forceinline__ void stage_group2(const uint4 (&raw)[2], uint4 (&o)[2], float& sum) {
  // raw: x of the group, natural order x0..x15 as 8 fp16 pairs
  const unsigned r[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
  sum = block_sum8({r[0], r[1], r[2], r[3]}) + block_sum8({r[4], r[5], r[6], r[7]});
  // pair p (0..7) = (x_p, x_{p+8}) scaled by 4^-(p%4)
  unsigned pr[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const unsigned lo = r[p >> 1], hi = r[4 + (p >> 1)];
    // x_p is the low (p even) or high (p odd) half of r[p/2]; x_{p+8} likewise of r[4 + p/2]
    pr[p] = __builtin_amdgcn_perm(hi, lo, (p & 1) ? 0x07060302u : 0x05040100u);
    const _Float16 sc = (p % 4 == 0) ? (_Float16)1.0f : ((p % 4 == 1) ? (_Float16)0.25f
                                                        : ((p % 4 == 2) ? (_Float16)0.0625f : (_Float16)0.015625f));
    if (p % 4) pr[p] = as_u(as_h2(pr[p]) * f16x2{sc, sc});
  }
  o[0] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
  o[1] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
}

// Sixteen 2-bit codes of a word -> 8 fp16 subnormal pairs in the order of stage_group2.
__device__ __forceinline__ void unpack16_2b(unsigned d, unsigned (&u)[8]) {
  const unsigned d8 = d >> 8;
  u[0] = d & 0x00030003u;
  u[1] = d & 0x000C000Cu;
  u[2] = d & 0x00300030u;
  u[3] = d & 0x00C000C0u;
  u[4] = d8 & 0x00030003u;
  u[5] = d8 & 0x000C000Cu;
  u[6] = d8 & 0x00300030u;
  u[7] = d8 & 0x00C000C0u;
}

template <int B, int JMAX, int R, int D>
__global__ void __launch_bounds__(64 * k2Waves) k_gemv_2b(const uint8_t* __restrict__ packed,
                                                         const __half* __restrict__ delta,
                                                         const __half* __restrict__ zero, int64_t N, int64_t K,
                                                         int out_dtype, const __half* __restrict__ x,
                                                         void* __restrict__ y) {
  static_assert(D >= 1 && D <= R, "rows in flight must be within the wave's rows");  // D: rows in flight
  constexpr bool XREG = B * JMAX <= 3;
  constexpr int NT = 64 * k2Waves;
  extern __shared__ float lds[];
  const int nch = (int)(K / 64);              // 64-code chunks per row
  const int ngr = (int)(K / 16);              // groups per row
  float* sg = lds;                            // [B][ngr] group sums of x
  uint4* xs = reinterpret_cast<uint4*>(sg + ((B * ngr + 3) & ~3));  // [B][8][nch] staged x
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t TW = 1;                                       // a wave's R rows are consecutive
  const int64_t gw = ((int64_t)blockIdx.x * k2Waves + wave) * R;  // its first row

  // 1. x: one group (32 bytes) per task
  constexpr int XR = (B * 64 * JMAX * 4 + NT - 1) / NT;
  const int ntask = B * ngr;
  uint4 xr[XR][2];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = min(tid + NT * i, ntask - 1);
    xr[i][0] = *reinterpret_cast<const uint4*>(x + 16 * idx);
    xr[i][1] = *reinterpret_cast<const uint4*>(x + 16 * idx + 8);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the first D rows: codes (16 B per chunk) and the four groups' steps and zeros (8 B each)
  uint4 wv[D][JMAX];
  uint2 dmv[D][JMAX], zmv[D][JMAX];
  auto issue = [&](int s, int64_t n) {
    const uint8_t* wrow = packed + n * (K / 4);
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      wv[s][j] = ld_stream16(wrow + 16 * c);
      dmv[s][j] = *reinterpret_cast<const uint2*>(delta + n * ngr + 4 * c);
      zmv[s][j] = *reinterpret_cast<const uint2*>(zero + n * ngr + 4 * c);
    }
  };
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, gw + s * TW);

  // 3. stage x: group gi of row m -> pieces xs[(m * 8 + 2 (gi % 4) + h) * nch + gi / 4]
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = min(tid + NT * i, ntask - 1);  // past the end: the last task again (same values)
    const int m = idx / ngr, gi = idx % ngr, c = gi / 4, t = gi % 4;
    uint4 o[2];
    float sum;
    stage_group2(xr[i], o, sum);
    xs[(m * 8 + 2 * t) * nch + c] = o[0];
    xs[(m * 8 + 2 * t + 1) * nch + c] = o[1];
    sg[m * ngr + gi] = sum;
  }
  lds_barrier();  // LDS hand-over; the weight loads stay in flight
  uint4 xq[XREG ? B : 1][XREG ? JMAX : 1][8];
  float sxr[B][JMAX][4];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int c = min(lane + 64 * j, nch - 1);
      if constexpr (XREG) {
#pragma unroll
        for (int pc = 0; pc < 8; ++pc) xq[b][j][pc] = xs[(b * 8 + pc) * nch + c];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sxr[b][j][t] = sg[b * ngr + 4 * c + t];
    }

  // 4. rows
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
      const unsigned dmw[2] = {dmv[s][j].x, dmv[s][j].y}, zmw[2] = {zmv[s][j].x, zmv[s][j].y};
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // group t of the chunk = word t
        unsigned u[8];
        unpack16_2b(dw[t], u);
        const unsigned short dh = (unsigned short)(dmw[t >> 1] >> (16 * (t & 1)));
        const unsigned short zh = (unsigned short)(zmw[t >> 1] >> (16 * (t & 1)));
        const float dl = valid ? __half2float(__ushort_as_half(dh)) * kSubScale : 0.f;
        const float zz = __half2float(__ushort_as_half(zh)) * kSubScaleInv;
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float P = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint4 xv;
            if constexpr (XREG)
              xv = xq[b][j][2 * t + h];
            else
              xv = xs[(b * 8 + 2 * t + h) * nch + c];
            const unsigned xu[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) P = __builtin_amdgcn_fdot2(as_h2(xu[e]), as_h2(u[4 * h + e]), P, false);
          }
          acc[b] = fmaf(dl, fmaf(-zz, sxr[b][j][t], P), acc[b]);
        }
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
// Axis 1, 3-bit (ten codes per 32-bit word over the flat index, so a row starts inside a word:
// code (n, k) is slot f mod 10 of word f / 10, f = nK + k).  A wave takes one row at a time;
// lane l takes the 8-code blocks m = l + 64j of the row (codes 8m .. 8m + 7, all in one group
// since g >= 16).  Their 24 bits lie in words q = f / 10 and q + 1 (f = nK + 8m): the 30-bit
// payloads concatenated into 64 bits and shifted right by 3 (f mod 10) put c0..c7 at bits
// 0..23; (v & 0xFFF) | ((v << 4) & 0xFFF0000) then gives the fp16 subnormal pairs (c0, c4),
// 8 (c1, c5), 64 (c2, c6) and, after >> 9, (c3, c7) with one AND each.  x is staged per block
// in that pair order with 1, 1/8, 1/64, 1 on the four slots, and the block sums of x beside
// it; per block acc += delta 2^24 (P - z 2^-24 S) (v_dot2_f32_f16, fp32 sums).
// ------------------------------------------------------------------------------------------
constexpr int k3Waves = 4;
constexpr int k3PadB = 4;  // zero blocks staged before and after x (a row's first and last superblock overhang)
constexpr int k3PadG = 2;  // zero groups before and after a row's metadata
// 16-byte blocks of x each thread loads: J superblocks per lane cover rows of K < 40 (64 J - 1)
// codes, i.e. fewer than 320 J blocks of 8, and K <= 8192 caps it at 1024 blocks
constexpr int x_loads_3b(int B, int J) { return (B * (320 * J < 1024 ? 320 * J : 1024) + 64 * k3Waves - 1) / (64 * k3Waves); }

// Four 16-byte aligned words hold 40 codes: five 8-code blocks whose bit positions are fixed
// (block 1 straddles words 0-1, block 2 words 1-2, block 3 words 2-3).  A row starts at code
// n*K, a multiple of 8, so every block lies inside one row and, with g >= 16 a multiple of 8,
// inside one group.  Lane i of a wave takes superblock sb0 + i + 64 j of its row, with sb0 the
// superblock holding the row's first code; blocks of a neighbouring row in the row's first and
// last superblock meet zero x and zero metadata.
template <int B, int J, int R>
__global__ void __launch_bounds__(64 * k3Waves) k_gemv_3b(const uint32_t* __restrict__ packed,
                                                         const __half* __restrict__ delta,
                                                         const __half* __restrict__ zero, int64_t N, int64_t K,
                                                         int gs_log2, int out_dtype, const __half* __restrict__ x,
                                                         void* __restrict__ y) {
  constexpr int D = R < 2 ? R : 2;  // rows in flight per wave
  extern __shared__ float lds3[];
  const int nb8 = (int)(K / 8);      // 8-code blocks per row
  const int xs = nb8 + 2 * k3PadB;   // staged blocks per batch row
  const int G = (int)(K >> gs_log2);  // groups per row
  const int gsr = G + 2 * k3PadG;
  float* sxb = lds3;                                              // [B][xs] block sums of x
  uint4* xq = reinterpret_cast<uint4*>(sxb + ((B * xs + 3) & ~3));  // [B][xs] staged x pairs
  float2* meta = reinterpret_cast<float2*>(xq + B * xs);          // [waves][R][gsr] (step 2^24, -zero 2^-24)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t TW = 1;                                       // a wave's R rows are consecutive
  const int64_t gw = ((int64_t)blockIdx.x * k3Waves + wave) * R;  // its first row
  const int64_t nwt = (N * K + 9) / 10;  // words of the tensor

  // 1. this thread's blocks of x and this wave's rows' metadata, ahead of the weight stream
  constexpr int XR = x_loads_3b(B, J);
  constexpr int MR = 3;  // metadata entries per lane and row loaded early: rows of up to 188 groups
  const int nxb = B * nb8;
  uint4 xr[XR];
#pragma unroll
  for (int t = 0; t < XR; ++t) {
    const int i = min(tid + 64 * k3Waves * t, nxb - 1);
    xr[t] = *reinterpret_cast<const uint4*>(x + 8 * (int64_t)i);  // x is [B][K] contiguous
  }
  unsigned dm[R][MR], zm[R][MR];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t gb = (gw + r * TW) * G;
#pragma unroll
    for (int t = 0; t < MR; ++t) {
      const int gi = min(max(lane + 64 * t - k3PadG, 0), G - 1);
      dm[r][t] = __half_as_ushort(delta[gb + gi]);
      zm[r][t] = __half_as_ushort(zero[gb + gi]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the first D rows' words, in flight
  uint4 wv[D][J];
  auto issue = [&](int s, int64_t n) {
    const int64_t f0 = n * K, sb0 = f0 / 40;
    const int nsb = (int)((f0 + K - 1) / 40 - sb0) + 1;
    const int lim = (int)min(nwt - 4 * sb0, (int64_t)INT_MAX);  // words from the row's first superblock on
    const int nfull = min(lim / 4, nsb);  // superblocks wholly inside the tensor: >= 1 as K >= 40
    const uint4* base = reinterpret_cast<const uint4*>(packed) + sb0;
#pragma unroll
    for (int j = 0; j < J; ++j) wv[s][j] = base[(unsigned)min(lane + 64 * j, nfull - 1)];
    if (nfull < nsb) {  // the tensor ends inside this row's last superblock: its words one by one
      const uint32_t* wp = packed + 4 * sb0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int i = lane + 64 * j;
        if (i >= nfull && i < nsb) {
          wv[s][j].x = wp[min(4 * i, lim - 1)];
          wv[s][j].y = wp[min(4 * i + 1, lim - 1)];
          wv[s][j].z = wp[min(4 * i + 2, lim - 1)];
          wv[s][j].w = wp[min(4 * i + 3, lim - 1)];
        }
      }
    }
  };
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, gw + s * TW);

  // 3. metadata as floats (step 2^24, -zero 2^-24), zero-padded at both ends of each row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float2* mr = meta + (wave * R + r) * gsr;
#pragma unroll
    for (int t = 0; t < MR; ++t) {
      const int i = lane + 64 * t, gi = i - k3PadG;
      float2 v = {0.f, 0.f};
      if (gi >= 0 && gi < G) {
        v.x = __half2float(__ushort_as_half((unsigned short)dm[r][t])) * kSubScale;
        v.y = -__half2float(__ushort_as_half((unsigned short)zm[r][t])) * kSubScaleInv;
      }
      if (i < gsr) mr[i] = v;
    }
    if (gsr > 64 * MR) {  // longer rows: the rest after the words (waits for them)
      const int64_t gb = (gw + r * TW) * G;
      for (int i = lane + 64 * MR; i < gsr; i += 64) {
        const int gi = i - k3PadG;
        float2 v = {0.f, 0.f};
        if (gi < G) {
          v.x = __half2float(delta[gb + gi]) * kSubScale;
          v.y = -__half2float(zero[gb + gi]) * kSubScaleInv;
        }
        mr[i] = v;
      }
    }
  }

  // 4. stage x: block m of batch row b as [(x0, x4), (x1, x5)/8, (x2, x6)/64, (x3, x7)] at
  //    b * xs + pad + m, and its sum; the pads are zero
#pragma unroll
  for (int t = 0; t < XR; ++t) {
    const int i = tid + 64 * k3Waves * t;
    if (i < nxb) {
      const int b = i / nb8, m = i - b * nb8;
      const uint4 raw = xr[t];
      const unsigned r4[4] = {raw.x, raw.y, raw.z, raw.w};
      uint4 o;
      o.x = __builtin_amdgcn_perm(raw.z, raw.x, 0x05040100u);  // x0 | x4 << 16
      o.y = as_u(as_h2(__builtin_amdgcn_perm(raw.z, raw.x, 0x07060302u)) *
                 f16x2{(_Float16)0.125f, (_Float16)0.125f});  // (x1, x5) / 8
      o.z = as_u(as_h2(__builtin_amdgcn_perm(raw.w, raw.y, 0x05040100u)) *
                 f16x2{(_Float16)0.015625f, (_Float16)0.015625f});  // (x2, x6) / 64
      o.w = __builtin_amdgcn_perm(raw.w, raw.y, 0x07060302u);  // x3 | x7 << 16
      sxb[b * xs + k3PadB + m] = block_sum8(r4);
      xq[b * xs + k3PadB + m] = o;
    }
  }
  if (tid < B * 2 * k3PadB) {
    const int b = tid / (2 * k3PadB), p = tid % (2 * k3PadB);
    const int m = p < k3PadB ? p : nb8 + p;  // pads before and after the row
    sxb[b * xs + m] = 0.f;
    xq[b * xs + m] = uint4{0u, 0u, 0u, 0u};
  }
  lds_barrier();

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = r % D;
    const int64_t n = gw + r * TW;
    const int64_t f0 = n * K, sb0 = f0 / 40;
    const int nsb = (int)((f0 + K - 1) / 40 - sb0) + 1;
    const int crow = (int)(5 * sb0 - f0 / 8) + k3PadB;  // staged index of the first superblock's block 0
    const float2* mr = meta + (wave * R + r) * gsr + k3PadG;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = lane + 64 * j;
      if (i < nsb) {
        const uint4 w = wv[s][j];
        const unsigned v[5] = {w.x, __builtin_amdgcn_ubfe(w.x, 24, 6) | (w.y << 6),
                               __builtin_amdgcn_ubfe(w.y, 18, 12) | (w.z << 12),
                               __builtin_amdgcn_ubfe(w.z, 12, 18) | (w.w << 18), w.w >> 6};
        const int m0 = crow + 5 * i;  // staged block index, in [0, nb8 + 2 pads)
#pragma unroll
        for (int bb = 0; bb < 5; ++bb) {
          const unsigned x0 = (v[bb] & 0x00000FFFu) | ((v[bb] << 4) & 0x0FFF0000u);
          const unsigned cp[4] = {x0 & 0x00070007u, x0 & 0x00380038u, x0 & 0x01C001C0u,
                                  (x0 >> 9) & 0x00070007u};
          const int m = m0 + bb;
          const float2 md = mr[(8 * (m - k3PadB)) >> gs_log2];
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const uint4 xv = xq[b * xs + m];
            float P = __builtin_amdgcn_fdot2(as_h2(xv.x), as_h2(cp[0]), 0.f, false);
            P = __builtin_amdgcn_fdot2(as_h2(xv.y), as_h2(cp[1]), P, false);
            P = __builtin_amdgcn_fdot2(as_h2(xv.z), as_h2(cp[2]), P, false);
            P = __builtin_amdgcn_fdot2(as_h2(xv.w), as_h2(cp[3]), P, false);
            acc[b] = fmaf(md.x, fmaf(md.y, sxb[b * xs + m], P), acc[b]);
          }
        }
      }
    }
    if (r + D < R) issue(s, gw + (r + D) * TW);
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
// launchers
// ------------------------------------------------------------------------------------------
size_t ax0_lds_bytes(int B, int64_t K) { return (size_t)4 * B * 4 + (size_t)B * K * 2; }

template <int B, int JMAX, int RPW>
hipError_t ax0_launch(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                      const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int subsets = g / (kAx0Waves * RPW);
  const dim3 grid((unsigned)((N / g) * subsets));
  hipLaunchKernelGGL((k_gemv_ax0<B, JMAX, RPW, 2>), grid, dim3(64 * kAx0Waves), ax0_lds_bytes(B, K), st, packed, delta,
                     zero, N, K, g, subsets, y_dtype, x, y);
  return hipGetLastError();
}

// rows per wave: a whole group's g rows per block where g allows (fewer blocks re-staging a)
template <int B, int JMAX>
hipError_t ax0_rpw(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                   const __half* x, void* y, int y_dtype, hipStream_t st) {
  if constexpr (B == 1 || JMAX <= 4)  // 32 unrolled rows of B = 2, K > 8192 run out of registers
    if (g >= 128) return ax0_launch<B, JMAX, 32>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
  if (g >= 64) return ax0_launch<B, JMAX, 16>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
  if (g == 32) return ax0_launch<B, JMAX, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
  return ax0_launch<B, JMAX, 4>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
}

template <int B>
hipError_t ax0_b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                 const __half* x, void* y, int y_dtype, hipStream_t st) {
  switch ((K / 32 + 63) / 64) {
    case 1: return ax0_rpw<B, 1>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 2: return ax0_rpw<B, 2>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 3: return ax0_rpw<B, 3>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 4: return ax0_rpw<B, 4>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 5:
    case 6: return ax0_rpw<B, 6>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    default: return ax0_rpw<B, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
  }
}

// two rows per wave, both in flight from the start (more rows per wave measured slower: the
// rows of a wave then queue behind each other's memory latency)
inline int rows_per_wave_2b(int64_t N) { return N % (2 * k2Waves) == 0 ? 2 : 1; }

size_t lds_2b(int B, int64_t K) { return (size_t)((B * (K / 16) + 3) & ~int64_t(3)) * 4 + (size_t)B * K * 2; }

template <int B, int JMAX>
hipError_t b2_j(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int R = rows_per_wave_2b(N);
  const dim3 grid((unsigned)(N / (R * k2Waves))), block(64 * k2Waves);
  const size_t lds = lds_2b(B, K);
  if (R == 2)
    hipLaunchKernelGGL((k_gemv_2b<B, JMAX, 2, 2>), grid, block, lds, st, packed, delta, zero, N, K, y_dtype, x, y);
  else
    hipLaunchKernelGGL((k_gemv_2b<B, JMAX, 1, 1>), grid, block, lds, st, packed, delta, zero, N, K, y_dtype, x, y);
  return hipGetLastError();
}

template <int B>
hipError_t b2_b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                const __half* x, void* y, int y_dtype, hipStream_t st) {
  switch ((K / 64 + 63) / 64) {
    case 1: return b2_j<B, 1>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 2: return b2_j<B, 2>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 3: return b2_j<B, 3>(packed, delta, zero, N, K, x, y, y_dtype, st);
    default: return b2_j<B, 4>(packed, delta, zero, N, K, x, y, y_dtype, st);
  }
}

// staged x (pairs and block sums, zero-padded) and the metadata of the block's rows
size_t lds_3b(int B, int R, int64_t K, int g) {
  const int64_t xs = K / 8 + 2 * k3PadB;
  return (size_t)((B * xs + 3) & ~int64_t(3)) * 4 + (size_t)B * xs * 16 + (size_t)k3Waves * R * (K / g + 2 * k3PadG) * 8;
}
inline int rows_per_wave_3b(int64_t N) { return N % (2 * k3Waves) == 0 ? 2 : 1; }

template <int B, int J>
hipError_t b3_r(const uint32_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gl,
                const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int R = rows_per_wave_3b(N);
  // every superblock of a row has a lane, every block of x a loading thread, every row a wave
  if (K < 40 || (K / 40 + 2) > 64 * J || B * (K / 8) > x_loads_3b(B, J) * 64 * k3Waves || N % (R * k3Waves) != 0)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(N / (R * k3Waves))), block(64 * k3Waves);
  const size_t lds = lds_3b(B, R, K, 1 << gl);
  if (R == 2)
    hipLaunchKernelGGL((k_gemv_3b<B, J, 2>), grid, block, lds, st, packed, delta, zero, N, K, gl, y_dtype, x, y);
  else
    hipLaunchKernelGGL((k_gemv_3b<B, J, 1>), grid, block, lds, st, packed, delta, zero, N, K, gl, y_dtype, x, y);
  return hipGetLastError();
}

// superblocks per lane: a row of K codes touches at most K/40 + 2 superblocks
template <int B>
hipError_t b3_j(const uint32_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int gl,
                const __half* x, void* y, int y_dtype, hipStream_t st) {
  switch ((K / 40 + 2 + 63) / 64) {
    case 1: return b3_r<B, 1>(packed, delta, zero, N, K, gl, x, y, y_dtype, st);
    case 2: return b3_r<B, 2>(packed, delta, zero, N, K, gl, x, y, y_dtype, st);
    case 3: return b3_r<B, 3>(packed, delta, zero, N, K, gl, x, y, y_dtype, st);
    default: return b3_r<B, 4>(packed, delta, zero, N, K, gl, x, y, y_dtype, st);
  }
}

}  // namespace

// 3-bit product: rows of at most 8192 codes (16 blocks of 8 per lane), K a multiple of 8
bool gemv_3b_supported(int64_t K, int g) {
  return K % 8 == 0 && K >= 40 && K <= 8192 && (g == 16 || g == 32 || g == 64 || g == 128 || g == 256);
}
size_t gemv_3b_lds_bytes(int64_t N, int64_t K, int g, int64_t batch) {
  return lds_3b((int)batch, rows_per_wave_3b(N), K, g);
}

hipError_t launch_gemv_3b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                          const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  int gl = 4;
  while ((1 << gl) < g) ++gl;
  return batch == 1 ? b3_j<1>(pk, delta, zero, N, K, gl, x, y, y_dtype, st)
                    : b3_j<2>(pk, delta, zero, N, K, gl, x, y, y_dtype, st);
}

// axis 0, batch 3..8: two strips per block where g and the block count allow
inline int mf0_strips(int64_t N, int g) { return (g % 32 == 0 && (N / g) * (g / 32) >= 256) ? 2 : 1; }

template <int B, int SPB, int NSEG, int W>
hipError_t mf0_launch(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                      const __half* x, void* y, int y_dtype, hipStream_t st) {
  const int subsets = g / (16 * SPB);
  const int xcd_map = (N / g) % 8 == 0;
  hipLaunchKernelGGL((k_gemv_mf0<B, SPB, NSEG, W>), dim3((unsigned)((N / g) * subsets)), dim3(64 * W),
                     2 * mf0_stage_bytes(B, SPB, W), st, packed, delta, zero, N, K, g, subsets, xcd_map, y_dtype, x, y);
  return hipGetLastError();
}

// Rows of up to 8192 codes: 8 waves, up to 8 segments of 1024 codes as a compile-time count (the
// axis-1 kernel's choice; 28672 x 8192 at batch 8 measured below); longer rows: 16 waves and
// 2048-code segments in a run-time loop.
template <int B, int SPB>
hipError_t mf0_seg(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                   const __half* x, void* y, int y_dtype, hipStream_t st) {
  switch ((K + 1023) / 1024) {
    case 1: return mf0_launch<B, SPB, 1, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 2: return mf0_launch<B, SPB, 2, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 3: return mf0_launch<B, SPB, 3, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 4: return mf0_launch<B, SPB, 4, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 5: return mf0_launch<B, SPB, 5, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 6: return mf0_launch<B, SPB, 6, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 7: return mf0_launch<B, SPB, 7, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 8: return mf0_launch<B, SPB, 8, 8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    default: return mf0_launch<B, SPB, 0, 16>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
  }
}

template <int B>
hipError_t mf0_b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K, int g,
                 const __half* x, void* y, int y_dtype, hipStream_t st) {
  return mf0_strips(N, g) == 2 ? mf0_seg<B, 2>(packed, delta, zero, N, K, g, x, y, y_dtype, st)
                               : mf0_seg<B, 1>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
}

size_t gemv_ax0_lds_bytes(int64_t K, int64_t batch) {
  return batch <= 2 ? ax0_lds_bytes((int)batch, K) : 2 * (size_t)mf0_stage_bytes((int)batch, 2, 16);
}
size_t gemv_2b_lds_bytes(int64_t K, int64_t batch) { return lds_2b((int)batch, K); }

hipError_t launch_gemv_ax0(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                           int g, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  switch (batch) {
    case 1: return ax0_b<1>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 2: return ax0_b<2>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 3: return mf0_b<3>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 4: return mf0_b<4>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 5: return mf0_b<5>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 6: return mf0_b<6>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 7: return mf0_b<7>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    case 8: return mf0_b<8>(packed, delta, zero, N, K, g, x, y, y_dtype, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_2b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  return batch == 1 ? b2_b<1>(packed, delta, zero, N, K, x, y, y_dtype, st)
                    : b2_b<2>(packed, delta, zero, N, K, x, y, y_dtype, st);
}

}  // namespace hqq
