// Fused dequantise + matrix product for large batches, split along K (page "HQQ 算法解读",
// section "从压缩文件到一次前向": unpack, (q - zero) * scale, x @ W_hat^T, with fp32
// accumulation).
//
// A batch of 256 against an 8192-row weight gives only 2M outputs: one block per compute
// unit then owns an 8192-output tile, too small to feed the matrix cores from LDS and L2 (the
// activations would be re-read 128 times).  Here a block owns a 256 (batch) x 128 (weight
// rows) tile over a quarter of K (whatever split brings the grid to >= 256 blocks), so every
// weight is dequantised once and the activations are read N / 128 times; the splits' fp32
// partial sums go to a caller-provided workspace and a second kernel adds them in split order
// (deterministic) into y.
//
// Block = 4 waves; wave w owns batch rows 64w .. 64w + 63 of the tile and all 128 weight rows
// (4 x 8 tiles of v_mfma_f32_16x16x32_f16).  Per 128-code chunk:
//   * W_hat of the block's 128 rows is dequantised once into LDS (double buffered): thread t
//     takes row t / 2, 64 codes, and forms fp16(c 2^-24 * (d 2^24) - z d) with the mixed
//     fp16/fp32 FMA (the code is a masked fp16 subnormal; z d is exact in fp32), one rounding
//     to fp32 and one to fp16;
//   * the activations go straight from global memory (L2) into the A operand registers (no
//     other wave reads them), one chunk ahead;
//   * the packed codes of chunk c + 2 are loaded while chunk c is multiplied.
// One barrier per chunk.
//
// The same kernel, transposed, computes the input gradient dX = dY @ W_hat: output columns k of
// the weight, contraction over its rows (the dequantised tile is stored transposed in LDS).

#include <type_traits>

#include "hqq_gemv_common.h"

namespace hqq {
namespace {

constexpr int kSkBM = 256;          // batch rows per block
constexpr int kSkBN = 128;          // weight rows per block
constexpr int kSkBK = 128;          // codes per chunk
// LDS row stride of the W_hat tile (halves): 16 halves of padding for the forward product and 8
// for the transposed tile (measured at 8192 x 8192, batch 256: forward 56.0-56.8 us against
// 57.7-58.2 with 8; the transposed stores and their swizzle prefer 8: 58.9-59.4 against 59.5-60.7)
template <bool TRANS>
constexpr int sk_row() { return kSkBK + (TRANS ? 8 : 16); }
constexpr size_t kSkLds = 2 * kSkBN * (kSkBK + 16) * sizeof(_Float16);  // the larger of the two
constexpr int kSkMulWaves = 4;      // multiplying waves, each 64 batch rows x all 128 weight rows
constexpr int kSkThreads = 512;     // and as many staging waves

// Stored formats the split GEMM stages (4-bit axis 1 has its group size as a template
// parameter; the others take log2 of it at run time).  kFmt4A0: 4-bit codes with axis-0 groups
// (weight row n uses metadata row n mod (N/g), one step and zero per column).
constexpr int kFmt4 = 0, kFmt2 = 2, kFmt3 = 3, kFmt4A0 = 4;

// TRANS = false: y [batch, N] = x [batch, K] @ W_hat^T (the forward product; output index n,
//   contraction over k).  TRANS = true: dX [batch, K] = dY [batch, N] @ W_hat (its input
//   gradient; output index k, contraction over the weight rows n).  W is [N, K] in both.
// The LDS tile always holds W_hat as [output index][contraction index]; the transposed form
// writes it with an XOR swizzle of 16-byte blocks (block ^ 4 (output >> 5)), which keeps both
// its dword stores and the 16-byte fragment reads free of bank conflicts.
//
// Two roles per block, two waves per SIMD: waves 0-3 multiply (A from the tiled activations,
// B from the LDS tile), waves 4-7 stage the weight tile (codes and metadata two chunks ahead,
// dequantisation, LDS stores).  A wave's memory counter completes in issue order, so a wave
// that issued both would wait for the slow weight stream (HBM) whenever it needs its next
// activations (L2); split by role, each waits only for its own stream.  Both roles pass the
// same barriers: one after the first tile is staged and one per chunk.
template <int FMT, int GS, bool DIRECT, bool TRANS>
__global__ void __launch_bounds__(kSkThreads) k_gemm_sk(const uint8_t* __restrict__ packed, const __half* __restrict__ delta,
                                                 const __half* __restrict__ zero, int64_t N, int64_t K, int S,
                                                 const u32x4* __restrict__ xt, int64_t MG, int64_t batch,
                                                 float* __restrict__ part, void* __restrict__ y, int out_dtype,
                                                 int xcd_map, int gs_log2) {
  extern __shared__ _Float16 wt[];  // [2][kSkBN][kSkRow]
  constexpr int kSkRow = sk_row<TRANS>();
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t NO = TRANS ? K : N, KC = TRANS ? N : K;  // output and contraction lengths
  // Block b of a row of the grid runs on XCD b mod 8 (round-robin dispatch).  With xcd_map,
  // the S splits get 8 / S XCDs each (S <= 8) or each XCD gets S / 8 splits, so one XCD's L2
  // holds only its splits' columns of x.
  int tile, split;
  {
    const int b = blockIdx.x, nb = gridDim.x;
    if (xcd_map) {
      const int xcd = b & 7, r = b >> 3;
      if (S <= 8) {
        const int per = 8 / S;
        split = xcd / per;
        tile = r * per + xcd % per;
      } else {
        const int per = S / 8;
        split = xcd * per + r % per;
        tile = r / per;
      }
    } else {
      tile = b % (nb / S);
      split = b / (nb / S);
    }
  }
  // split s takes pairs of chunks [s C2 / S, (s + 1) C2 / S) of the C2 = KC / 256 pairs (S <= C2)
  const int64_t C2 = KC / (2 * kSkBK), p_lo = split * C2 / S, p_hi = (split + 1) * C2 / S;
  const int64_t n0 = (int64_t)tile * kSkBN, m0 = (int64_t)blockIdx.y * kSkBM, k0 = p_lo * 2 * kSkBK;
  const int nch = (int)(2 * (p_hi - p_lo));  // even, >= 2

  if constexpr (FMT != kFmt4) {
    if (wave >= kSkMulWaves) {
      // ---------------------------------------------------------------- staging waves, 2/3-bit
      // Forward: thread -> weight rows wr and 64 + wr, codes 32 wq .. 32 wq + 31 of each chunk.
      // Transposed: thread -> weight rows 2 wr and 2 wr + 1 of the chunk (contraction), codes
      // 32 wq .. +31 of the tile's output columns.  Either way 32 codes of one row from flat code
      // index f = n K + k, an even number (K % 128 == 0): 2-bit: 8 bytes; 3-bit: ten codes per
      // word, the 32 codes start at an even slot ph <= 8 of word f / 10 and end inside the fourth
      // word; 4-bit axis 0: 16 bytes, with the 32 steps and zeros of metadata row n mod (N / g)
      // at the same columns (64 bytes each).  Axis 1 with g = 16: codes 0..15 and 16..31 are two
      // groups; otherwise one.
      const int st = tid - 64 * kSkMulWaves;
      const int wr = st >> 2, wq = st & 3;
      _Float16* wdst = wt + wr * kSkRow + 32 * wq;
      int64_t fr[2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        fr[p] = TRANS ? (k0 + 2 * wr + p) * K + n0 + 32 * wq : (n0 + wr + 64 * p) * K + k0 + 32 * wq;
      const int64_t fstep = TRANS ? (int64_t)kSkBK * K : kSkBK;  // the next chunk
      constexpr int MD = FMT == kFmt4A0 ? 16 : 2;  // metadata dwords per row (axis 0: 32 fp16 each)
      struct Regs {
        unsigned w[2][4], dm[2][MD], zm[2][MD];
        int ph[2];
      };
      // axis 0: the thread's rows and first column; metadata index (n mod R0) K + k, R0 = N / g
      const unsigned R0 = (unsigned)(N >> gs_log2);
      unsigned mrow[2], mcol[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        mrow[p] = (unsigned)(TRANS ? k0 + 2 * wr + p : n0 + wr + 64 * p);
        mcol[p] = (unsigned)(TRANS ? n0 + 32 * wq : k0 + 32 * wq);
      }
      auto load_w = [&](int c, Regs& r) {
        const int64_t cc = min(c, nch - 1);  // past the end: reload the last chunk (never used)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int64_t f0 = fr[p] + fstep * cc;
          if constexpr (FMT == kFmt4A0) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(packed + f0 / 2);
            const unsigned row = mrow[p] + (TRANS ? (unsigned)(kSkBK * cc) : 0u);
            const unsigned col = mcol[p] + (TRANS ? 0u : (unsigned)(kSkBK * cc));
            const int64_t mi = (int64_t)(row % R0) * K + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              r.w[p][i] = v[i];
              const u32x4 dv = *reinterpret_cast<const u32x4*>(delta + mi + 8 * i);
              const u32x4 zv = *reinterpret_cast<const u32x4*>(zero + mi + 8 * i);
#pragma unroll
              for (int e = 0; e < 4; ++e) r.dm[p][4 * i + e] = dv[e], r.zm[p][4 * i + e] = zv[e];
            }
            continue;
          } else if constexpr (FMT == kFmt3) {
            const int64_t q0 = f0 / 10;
            r.ph[p] = (int)(f0 - 10 * q0);
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(packed) + q0;
#pragma unroll
            for (int i = 0; i < 4; ++i) r.w[p][i] = pw[i];
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(packed + f0 / 4);
            r.w[p][0] = v.x, r.w[p][1] = v.y;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int64_t gi = (f0 + 16 * h) >> gs_log2;
            r.dm[p][h] = __half_as_ushort(delta[gi]);
            r.zm[p][h] = __half_as_ushort(zero[gi]);
          }
        }
      };
      // W_hat of the thread's 32 codes of row p, natural order: blocks of 8 codes (4 dwords of pairs)
      auto decode = [&](const Regs& r, int p, u32x4 (&o)[4]) {
        if constexpr (FMT == kFmt4A0) {
          // dword t: codes 8t..8t+7 as fp16 subnormals (c0, c4), (16 c1, 16 c5), (c2, c6),
          // (16 c3, 16 c7); each code with its own step and zero: fp16(c 2^-24 (d S) - z d),
          // S = 2^24 (2^20 for the odd codes), z d exact in fp32
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const unsigned dw = r.w[p][t];
            const f16x2 P[4] = {as_h2(dw & 0x000F000Fu), as_h2(dw & 0x00F000F0u), as_h2((dw >> 8) & 0x000F000Fu),
                                as_h2((dw >> 8) & 0x00F000F0u)};
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float c = (float)P[e & 3][e >> 2];
              const f16x2 dp = as_h2(r.dm[p][4 * t + (e >> 1)]), zp = as_h2(r.zm[p][4 * t + (e >> 1)]);
              const float d = (float)dp[e & 1], z = (float)zp[e & 1];
              w[e] = __builtin_fmaf(c, d * ((e & 1) ? 1048576.0f : 16777216.0f), -(z * d));
            }
            o[t] = u32x4{as_u(f16x2{(_Float16)w[0], (_Float16)w[1]}), as_u(f16x2{(_Float16)w[2], (_Float16)w[3]}),
                         as_u(f16x2{(_Float16)w[4], (_Float16)w[5]}), as_u(f16x2{(_Float16)w[6], (_Float16)w[7]})};
          }
          return;
        }
        float zd[2], d[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          d[h] = __half2float(__ushort_as_half((unsigned short)r.dm[p][h]));
          zd[h] = __half2float(__ushort_as_half((unsigned short)r.zm[p][h])) * d[h];
        }
        if constexpr (FMT == kFmt2) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float ds[4] = {d[h] * 16777216.0f, d[h] * 4194304.0f, d[h] * 1048576.0f, d[h] * 262144.0f};
            wq16_2b(r.w[p][h], ds, zd[h], o[2 * h], o[2 * h + 1]);
          }
        } else {
          decode32_3b(r.w[p], r.ph[p], d, zd, o);
        }
      };
      auto stage = [&](int buf, const Regs& r) {
        if constexpr (TRANS) {
          // the two rows' values of one output column paired into a dword (contraction 2 wr, 2 wr + 1),
          // 16-byte blocks swizzled as in the 4-bit path
          u32x4 r0[4], r1[4];
          decode(r, 0, r0);
          decode(r, 1, r1);
          _Float16* base = wt + buf * (kSkBN * kSkRow);
#pragma unroll
          for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int o = 32 * wq + 8 * sb + e;
              const unsigned v =
                  __builtin_amdgcn_perm(r1[sb][e >> 1], r0[sb][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
              const int blk = (wr >> 2) ^ (4 * (o >> 5));
              *reinterpret_cast<unsigned*>(base + o * kSkRow + 8 * blk + 2 * (wr & 3)) = v;
            }
        } else {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            u32x4 o[4];
            decode(r, p, o);
            _Float16* dst = wdst + buf * (kSkBN * kSkRow) + p * 64 * kSkRow;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) *reinterpret_cast<u32x4*>(dst + 8 * sb) = o[sb];
          }
        }
      };
      Regs ra, rb;
      load_w(0, ra);
      load_w(1, rb);
      stage(0, ra);
      load_w(2, ra);
      lds_barrier();
      for (int c = 0; c < nch; c += 2) {
        stage(1, rb);  // chunk c + 1 (always < nch: nch is even)
        load_w(c + 3, rb);
        lds_barrier();
        if (c + 2 < nch) stage(0, ra);  // chunk c + 2
        load_w(c + 4, ra);
        lds_barrier();
      }
      return;
    }
  } else {
    if (wave >= kSkMulWaves) {
      // ---------------------------------------------------------------- staging waves, 4-bit
      // Forward: thread -> weight rows wr and 64 + wr (output rows of the tile), codes
      // 32 wq .. 32 wq + 31 of each chunk.  Transposed: thread -> weight rows 2 wr and 2 wr + 1 of
      // the chunk (contraction), codes 32 wq .. +31 of the tile's output columns.  16 bytes per
      // row: one load instruction of a wave spans 16 (32) rows (each row of a 4-bit weight with
      // K = 8192 is its own 4 KB page, and an instruction's distinct pages are translated one
      // after another)
      const int st = tid - 64 * kSkMulWaves;
      const int wr = st >> 2, wq = st & 3;
      const int64_t G_row = K / GS;  // groups per weight row
      const uint8_t* wsrc;
      const __half *dsrc, *zsrc;
      int64_t wstride, mstride, wchunk, mchunk;
      if constexpr (TRANS) {
        wsrc = packed + (k0 + 2 * wr) * (K / 2) + (n0 + 32 * wq) / 2;
        dsrc = delta + (k0 + 2 * wr) * G_row + (n0 + 32 * wq) / GS;
        zsrc = zero + (k0 + 2 * wr) * G_row + (n0 + 32 * wq) / GS;
        wstride = K / 2, mstride = G_row;                                   // the second row
        wchunk = (int64_t)kSkBK * (K / 2), mchunk = (int64_t)kSkBK * G_row;  // the next chunk of rows
      } else {
        wsrc = packed + (n0 + wr) * (K / 2) + k0 / 2 + 16 * wq;
        dsrc = delta + (n0 + wr) * G_row + (k0 + 32 * wq) / GS;
        zsrc = zero + (n0 + wr) * G_row + (k0 + 32 * wq) / GS;
        wstride = 64 * (K / 2), mstride = 64 * G_row;  // the second row pass
        wchunk = kSkBK / 2, mchunk = kSkBK / GS;        // the next 128 codes
      }
      _Float16* wdst = wt + wr * kSkRow + 32 * wq;

      auto load_w = [&](int c, u32x4 (&wv)[2], unsigned (&dm)[2], unsigned (&zm)[2]) {
        const int cc = min(c, nch - 1);  // past the end: reload the last chunk (never used)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          wv[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc + p * wstride + cc * wchunk));
          dm[p] = __half_as_ushort(dsrc[p * mstride + cc * mchunk]);
          zm[p] = __half_as_ushort(zsrc[p * mstride + cc * mchunk]);
        }
      };
      // the thread's share of one chunk -> LDS buffer `buf`, with the dequantisation constants of
      // its rows' groups: z d and d 2^24, d 2^20 (all exact).  Forward: 16-byte stores.
      // Transposed: the two rows' values of one output column paired into a dword.
      auto stage = [&](int buf, const u32x4 (&wv)[2], const unsigned (&dm)[2], const unsigned (&zm)[2]) {
        float zd[2], ds24[2], ds20[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float d = __half2float(__ushort_as_half((unsigned short)dm[p]));
          const float z = __half2float(__ushort_as_half((unsigned short)zm[p]));
          zd[p] = z * d, ds24[p] = d * 16777216.0f, ds20[p] = d * 1048576.0f;
        }
        _Float16* base = wt + buf * (kSkBN * kSkRow);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (TRANS) {
            const u32x4 r0 = wq8(wv[0][s], ds24[0], ds20[0], zd[0]);
            const u32x4 r1 = wq8(wv[1][s], ds24[1], ds20[1], zd[1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int o = 32 * wq + 8 * s + e;  // output column in the tile; contraction 2 wr, 2 wr + 1
              const unsigned v = __builtin_amdgcn_perm(r1[e >> 1], r0[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
              const int blk = (wr >> 2) ^ (4 * (o >> 5));
              *reinterpret_cast<unsigned*>(base + o * kSkRow + 8 * blk + 2 * (wr & 3)) = v;
            }
          } else {
            const int p = s >> 1, h = s & 1;
            _Float16* dst = wdst + buf * (kSkBN * kSkRow) + p * 64 * kSkRow;
#pragma unroll
            for (int i = 2 * h; i < 2 * h + 2; ++i)
              *reinterpret_cast<u32x4*>(dst + 8 * i) = wq8(wv[p][i], ds24[p], ds20[p], zd[p]);
          }
        }
      };

      // chunk c + 1 is staged while the multiplying waves use chunk c; the codes of chunk c + 3
      // are requested right after, so each wait covers codes requested two chunks earlier
      u32x4 wa[2], wb[2];
      unsigned dma[2], zma[2], dmb[2], zmb[2];
      load_w(0, wa, dma, zma);
      load_w(1, wb, dmb, zmb);
      stage(0, wa, dma, zma);
      load_w(2, wa, dma, zma);
      lds_barrier();
      for (int c = 0; c < nch; c += 2) {
        stage(1, wb, dmb, zmb);  // chunk c + 1 (always < nch: nch is even)
        load_w(c + 3, wb, dmb, zmb);
        lds_barrier();
        if (c + 2 < nch) stage(0, wa, dma, zma);  // chunk c + 2
        load_w(c + 4, wa, dma, zma);
        lds_barrier();
      }
      return;
    }
  }

  // ---------------------------------------------------------------- multiplying waves
  // A operand from the tiled copy of x: the 16 x 32 fragment of row group mg and k-step q is
  // 1 KB at xt[(q MG + mg) 64 ..], already in lane order (lane l: row l & 15, codes
  // 8 (l >> 4) .. +7), so every A load instruction reads one contiguous 1 KB
  const u32x4* xa[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) xa[t] = xt + ((k0 / 32) * MG + (m0 + 64 * wave + 16 * t) / 16) * 64 + lane;
  const int nsteps = 4 * nch;
  const int64_t astep = MG * 64;  // one k-step further in the tiled copy
  // 16-row batch tiles of this wave that hold rows of the batch (wave-uniform), rounded up to
  // 0, 1 or 4: the MFMAs and A loads of the others are skipped (small batches: the tile's rows
  // are mostly padding); the count is a compile-time constant, so the loops stay straight-line
  const int tmax = (int)max<int64_t>(0, min<int64_t>(4, (batch - (m0 + 64 * wave) + 15) / 16));
  // A operand of k-step q (32 codes) into one of four register slots
  auto load_a = [&](int q, u32x4 (&av)[4], auto tm) {
    const int64_t off = (int64_t)min(q, nsteps - 1) * astep;
#pragma unroll
    for (int t = 0; t < decltype(tm)::value; ++t) av[t] = xa[t][off];
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk from LDS buffer `buf`.  k-step s: MFMAs in fragment order j (four batch tiles
  // each); fragment j's registers are refilled from LDS with k-step s + 1 right after its four
  // MFMAs; A slot s is refilled with k-step s of the next chunk after its last MFMA (A runs a
  // chunk ahead).  The scheduling barriers keep the loads where they are written (the
  // compiler would otherwise sink them to the loop end and wait for them there).
  u32x4 as[4][4];
  const _Float16* src0 = wt + (lane & 15) * kSkRow + 8 * (lane >> 4);
  auto chunk = [&](int buf, int c, auto tm) {
    const _Float16* src = src0 + buf * (kSkBN * kSkRow);
    // fragment j, k-step s: 16-byte block 4s + (lane >> 4) of its row (swizzled when TRANS)
    auto bfrag = [&](int j, int s) {
      const int sb = TRANS ? (s ^ (j >> 1)) : s;
      return *reinterpret_cast<const f16x8*>(src + 16 * j * kSkRow + 32 * sb);
    };
    f16x8 B[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) B[j] = bfrag(j, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int t = 0; t < decltype(tm)::value; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, as[s][t]), B[j], acc[t][j], 0, 0, 0);
        if (s < 3) B[j] = bfrag(j, s + 1);
      }
      load_a(4 * c + s + 4, as[s], tm);  // into the registers just read: no copy at the loop edge
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto run = [&](auto tm) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) load_a(s4, as[s4], tm);
    lds_barrier();  // the first tile is staged
    for (int c = 0; c < nch; c += 2) {
      if constexpr (decltype(tm)::value > 0) chunk(0, c, tm);
      lds_barrier();
      if constexpr (decltype(tm)::value > 0) chunk(1, c + 1, tm);
      lds_barrier();
    }
  };
  if (tmax > 1)
    run(std::integral_constant<int, 4>{});
  else if (tmax == 1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});

  // D layout: acc[t][j][r] is batch row 64 wave + 16 t + 4 (lane >> 4) + r, weight row
  // 16 j + (lane & 15)
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 64 * wave + 16 * t + 4 * (lane >> 4) + r;
      if (m >= batch) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t n = n0 + 16 * j + (lane & 15);
        if constexpr (DIRECT) {
          if (out_dtype == HQQ_OUT_F16)
            store_y<HQQ_OUT_F16>(y, m * NO + n, acc[t][j][r]);
          else
            store_y<HQQ_OUT_F32>(y, m * NO + n, acc[t][j][r]);
        } else {
          part[((int64_t)split * batch + m) * NO + n] = acc[t][j][r];
        }
      }
    }
}


// y = sum over the splits of the partial sums, in split order; 4 outputs per thread.
__global__ void __launch_bounds__(256) k_splitk_sum(const float* __restrict__ part, int S, int64_t MN,
                                                    void* __restrict__ y, int out_dtype) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
  for (int k = 1; k < S; ++k) s += *reinterpret_cast<const f32x4*>(part + (int64_t)k * MN + i);
  if (out_dtype == HQQ_OUT_F16) {
    const f16x2 a = {(_Float16)s[0], (_Float16)s[1]}, b = {(_Float16)s[2], (_Float16)s[3]};
    *reinterpret_cast<uint2*>(reinterpret_cast<__half*>(y) + i) = make_uint2(as_u(a), as_u(b));
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + i) = s;
  }
}

// x [batch, K] -> xt: for k-step q (32 codes) and row group mg (16 rows), 64 lanes x 16 bytes,
// lane l holding row 16 mg + (l & 15) (rows past the batch repeat the last row), codes
// 32 q + 8 (l >> 4) .. +7.  A block moves a 16-row x 512-code tile through LDS: it reads
// 1 KB row pieces and writes sixteen whole 1 KB fragments (the last tile of a row may hold
// 256 codes: eight fragments).
constexpr int kTileCols = 512;
__global__ void __launch_bounds__(256) k_tile_x(const __half* __restrict__ x, int64_t batch, int64_t K, int64_t MG,
                                                u32x4* __restrict__ xt) {
  __shared__ u32x4 tile[16][kTileCols / 8 + 1];
  const int tid = threadIdx.x;
  const int64_t mg = blockIdx.y, c0 = (int64_t)blockIdx.x * kTileCols;
  const int pieces = (int)min<int64_t>(kTileCols, K - c0) / 8;  // 16-byte pieces of a row in the tile
  {
    const int r = tid >> 4, cp = (tid & 15) * 4;  // row, first 16-byte piece of four
    const int64_t src_row = min(16 * mg + r, batch - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + src_row * K + c0) + cp;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (cp + i < pieces) tile[r][cp + i] = src[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, qb = e >> 6, l = e & 63;
    if (4 * qb < pieces) xt[((c0 / 32 + qb) * MG + mg) * 64 + l] = tile[l & 15][4 * qb + (l >> 4)];
  }
}

}  // namespace

// Splits of K for the split GEMM: the smallest power of two that brings the grid to >= 256
// blocks while every split keeps >= 1 pair of 128-code chunks (the K / 256 pairs are dealt out
// as evenly as they go: K = 11008 in 8 splits gives splits of 5 and 6 pairs).  0 = not applicable.
int gemm_splits(int64_t N, int64_t K, int64_t batch) {
  if (N % kSkBN != 0 || K % (2 * kSkBK) != 0 || batch <= 0) return 0;
  const int64_t tiles = (N / kSkBN) * ((batch + kSkBM - 1) / kSkBM), C2 = K / (2 * kSkBK);
  int S = 1;
  while (tiles * S < 256 && 2 * S <= C2) S *= 2;
  return S;
}

namespace {
size_t tiled_x_bytes(int64_t K, int64_t batch) {
  const int64_t MG = (batch + kSkBM - 1) / kSkBM * (kSkBM / 16);  // whole blocks of batch rows
  return ((size_t)MG * 16 * (size_t)K * 2 + 255) & ~size_t(255);
}
}  // namespace

size_t gemm_workspace_bytes(int64_t N, int64_t K, int64_t batch) {
  const int S = gemm_splits(N, K, batch);
  if (S == 0) return 0;
  return tiled_x_bytes(K, batch) + (S > 1 ? (size_t)S * (size_t)batch * (size_t)N * sizeof(float) : 0);
}

namespace {
// One split product: tile the A operand (x, or dY for the input gradient) into fragments, the
// split GEMM, and the sum over splits.  NO = output length (N, or K), KC = contraction (K, or N).
template <int FMT, int GS, bool DIRECT, bool TRANS>
void launch_sk(dim3 grid, hipStream_t st, const uint8_t* packed, const __half* delta, const __half* zero, int64_t N,
               int64_t K, int S, const u32x4* xt, int64_t MG, int64_t batch, float* pw, void* out, int y_dtype,
               int xcd_map, int gl) {
  hipLaunchKernelGGL((k_gemm_sk<FMT, GS, DIRECT, TRANS>), grid, dim3(kSkThreads), kSkLds, st, packed, delta, zero, N, K,
                     S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
}

template <bool DIRECT, bool TRANS>
void launch_fmt(int fmt, int gs, dim3 grid, hipStream_t st, const uint8_t* packed, const __half* delta,
                const __half* zero, int64_t N, int64_t K, int S, const u32x4* xt, int64_t MG, int64_t batch,
                float* pw, void* out, int y_dtype, int xcd_map) {
  int gl = 0;
  while ((1 << gl) < gs) ++gl;
  if (fmt == kFmt4A0) {
    launch_sk<kFmt4A0, 0, DIRECT, TRANS>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    return;
  }
  if constexpr (TRANS) {
    if (fmt == kFmt3)
      launch_sk<kFmt3, 0, DIRECT, true>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else if (fmt == kFmt2)
      launch_sk<kFmt2, 0, DIRECT, true>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else if (gs == 64)
      launch_sk<kFmt4, 64, DIRECT, true>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else
      launch_sk<kFmt4, 128, DIRECT, true>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
  } else {
    if (fmt == kFmt3)
      launch_sk<kFmt3, 0, DIRECT, false>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else if (fmt == kFmt2)
      launch_sk<kFmt2, 0, DIRECT, false>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else if (gs == 64)
      launch_sk<kFmt4, 64, DIRECT, false>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
    else
      launch_sk<kFmt4, 128, DIRECT, false>(grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map, gl);
  }
}

template <bool TRANS>
hipError_t launch_split(int fmt, const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                        int gs, const __half* a, int64_t batch, void* y, int y_dtype, void* workspace, hipStream_t st) {
  const int64_t NO = TRANS ? K : N, KC = TRANS ? N : K;
  const int S = gemm_splits(NO, KC, batch);
  const int64_t MG = (batch + kSkBM - 1) / kSkBM * (kSkBM / 16);
  u32x4* xt = reinterpret_cast<u32x4*>(workspace);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + tiled_x_bytes(KC, batch));
  hipLaunchKernelGGL(k_tile_x, dim3((unsigned)((KC + kTileCols - 1) / kTileCols), (unsigned)MG), dim3(256), 0, st, a,
                     batch, KC, MG, xt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = (NO / kSkBN) * S;  // blocks in a row of the grid: output tiles x splits
  const int xcd_map = nb % 8 == 0 && (S <= 8 ? (NO / kSkBN) % (8 / S) == 0 : S % 8 == 0);
  const dim3 grid((unsigned)nb, (unsigned)((batch + kSkBM - 1) / kSkBM));
  void* out = S == 1 ? y : nullptr;
  float* pw = S == 1 ? nullptr : part;
  if (S == 1) {
    launch_fmt<true, TRANS>(fmt, gs, grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map);
    return hipGetLastError();
  }
  launch_fmt<false, TRANS>(fmt, gs, grid, st, packed, delta, zero, N, K, S, xt, MG, batch, pw, out, y_dtype, xcd_map);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t MN = batch * NO;
  hipLaunchKernelGGL(k_splitk_sum, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, st, part, S, MN, y, y_dtype);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_split(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                             int gs, const __half* x, int64_t batch, void* y, int y_dtype, void* workspace,
                             hipStream_t st) {
  return launch_split<false>(kFmt4, packed, delta, zero, N, K, gs, x, batch, y, y_dtype, workspace, st);
}

hipError_t launch_gemm_fmt(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                           int nbits, int gs, int axis, const __half* x, int64_t batch, void* y, int y_dtype,
                           void* workspace, hipStream_t st) {
  const int fmt = axis == 0 ? kFmt4A0 : nbits == 3 ? kFmt3 : nbits == 2 ? kFmt2 : kFmt4;
  return launch_split<false>(fmt, packed, delta, zero, N, K, gs, x, batch, y, y_dtype, workspace, st);
}

hipError_t launch_gemm_dx(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          int nbits, int gs, int axis, const __half* dy, int64_t batch, void* dx, int dx_dtype,
                          void* workspace, hipStream_t st) {
  const int fmt = axis == 0 ? kFmt4A0 : nbits == 3 ? kFmt3 : nbits == 2 ? kFmt2 : kFmt4;
  return launch_split<true>(fmt, packed, delta, zero, N, K, gs, dy, batch, dx, dx_dtype, workspace, st);
}

}  // namespace hqq
