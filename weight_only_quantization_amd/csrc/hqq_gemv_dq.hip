// Fused product for small batches (3 to 16 rows of x) with 2-, 3- and 4-bit codes, axis-1
// groups, on the matrix units (page "HQQ 算法解读", section "从压缩文件到一次前向": unpack,
// (q - zero) * scale, x @ W_hat^T, fp32 accumulation; "为什么一定要分组" for the containers).
//
// A batch of up to 16 is one row tile of v_mfma_f32_16x16x32_f16, so the matrix units do the
// contraction at any such batch for the price of one (the dot-product path costs a multiply
// per code and batch row).  Each lane dequantises its weight codes to fp16 W_hat in registers
// with the same decoders as the split GEMM's staging (one mixed fp16/fp32 FMA per code) and
// hands them to the MFMA as its B operand; the activations are the A operand, read straight
// from global memory (x is a few hundred KB and stays in L2).  There is no LDS staging and no
// barrier in the main loop.
//
// Mapping.  A block owns kDqStrips strips of 16 weight rows (B-operand column n = lane % 16 of
// a strip is weight row n; one strip measured fastest: 11008 x 4096 at batch 8, 3-bit 17.3 us
// against 21.2 with two strips, whose 344 blocks of 8 waves fill 256 compute units in 1.3
// rounds) and splits the K / 128 chunks of 128 codes among its 8 waves in contiguous runs.  In a chunk, lane group h = lane / 16 takes codes 32h .. 32h + 31 of its row
// (16 bytes at 4 bits, 8 at 2 bits, four ten-code words at 3 bits), which are its B operands of
// the chunk's four k-steps (k-step s: codes 32h + 8s .. +7); the A operand of lane (m, h) at
// k-step s is x[m][128c + 32h + 8s .. +7], rows m past the batch reading the last row (their
// results are never stored).  The codes and metadata run several chunks ahead of their use,
// the activations one; the loop is unrolled to a compile-time chunk count per wave (chunks
// past a wave's run load a valid chunk and are dequantised with a zero step, so they add
// zeros).  At the end the waves' partial sums of each output are added in wave order through
// LDS (deterministic).

#include "hqq_gemv_common.h"

namespace hqq {
namespace {

constexpr int kDqStrips = 1;              // 16-row strips per block
constexpr int kDqRows = 16 * kDqStrips;    // weight rows per block
constexpr int kDqMaxWaves = 8;             // waves per block
constexpr int kDqAhead = 3;                // chunks of codes and activations in flight ahead of their use

template <int FMT, int NCW, bool EXACT>
__global__ void __launch_bounds__(64 * kDqMaxWaves) k_gemv_dq(const uint8_t* __restrict__ packed,
                                                              const __half* __restrict__ delta,
                                                              const __half* __restrict__ zero, int64_t N, int64_t K,
                                                              int gs_log2, const __half* __restrict__ x, int64_t batch,
                                                              void* __restrict__ y, int out_dtype) {
  static_assert(FMT == 2 || FMT == 3 || FMT == 4, "2-, 3- or 4-bit codes");
  constexpr int RING = kDqAhead + 1;
  constexpr int SP = kDqStrips;
  __shared__ f32x4 red[kDqMaxWaves * SP * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = (int)(blockDim.x >> 6);
  const int nl = lane & 15, h = lane >> 4;
  const int64_t C = K / 128;  // chunks per row
  // this wave's run of chunks: EXACT, every run is NCW chunks (C = NCW nw); otherwise at most NCW,
  // and chunk i of the run reads chunk max(0, min(i, nrun - 1)) past its end (c_lo < C, so a
  // valid one even for an empty run)
  const int64_t c_lo = EXACT ? (int64_t)wave * NCW : wave * C / nw;
  const int nrun = EXACT ? NCW : (int)((wave + 1) * C / nw - c_lo);
  const int64_t r0 = (int64_t)blockIdx.x * kDqRows;
  // per strip: flat index of the lane's first code in the run's first chunk (rows past N: the
  // last row), and the pointers the run's loads step from
  int64_t f_first[SP];
  const uint8_t* pc[SP];      // 2-/4-bit: byte of the lane's first code
  const uint32_t* pq[SP];     // 3-bit: word of the lane's first code
  int ph_first[SP];           // 3-bit: its slot in that word
  const __half *pd[SP], *pz[SP];  // step and zero of its group
#pragma unroll
  for (int p = 0; p < SP; ++p) {
    f_first[p] = min(r0 + 16 * p + nl, N - 1) * K + 32 * h + 128 * c_lo;
    pc[p] = packed + f_first[p] * FMT / 8;
    const int64_t q = f_first[p] / 10;
    pq[p] = reinterpret_cast<const uint32_t*>(packed) + q;
    ph_first[p] = (int)(f_first[p] - 10 * q);
    pd[p] = delta + (f_first[p] >> gs_log2);
    pz[p] = zero + (f_first[p] >> gs_log2);
  }
  const __half* xrow = x + min<int64_t>(nl, batch - 1) * K + 32 * h + 128 * c_lo;

  // ---- one chunk's loads: codes, and the step and zero of the lane's group (with groups of 16,
  //      of its two groups)
  struct WRegs {
    unsigned w[SP][4];
    unsigned dm[SP], zm[SP];
    int ph[SP];  // 3-bit: slot of the first code in w[p][0]
    bool valid;  // the chunk is in this wave's run
  };
  auto load_w = [&](int i, WRegs& r) {
    r.valid = EXACT || i < nrun;
    const int ci = EXACT ? i : max(0, min(i, nrun - 1));  // chunk of the run (an empty run: its first)
#pragma unroll
    for (int p = 0; p < SP; ++p) {
      if constexpr (FMT == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pc[p] + 64 * ci));
#pragma unroll
        for (int e = 0; e < 4; ++e) r.w[p][e] = v[e];
      } else if constexpr (FMT == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(pc[p] + 32 * ci);
        r.w[p][0] = v.x, r.w[p][1] = v.y, r.w[p][2] = 0u, r.w[p][3] = 0u;
      } else {
        // 128 codes = 12 words and 8 slots: chunk ci starts at slot ph_first + 8 ci of word
        // q_first + 12 ci (carried into the word index past slot 9)
        int slot = ph_first[p] + (EXACT ? (8 * i) % 10 : 8 * ci);
        int carry = EXACT ? (slot >= 10) : slot / 10;
        slot -= 10 * carry;
        r.ph[p] = slot;
        const uint32_t* pw = pq[p] + (EXACT ? 12 * i + (8 * i) / 10 : 12 * ci) + carry;
#pragma unroll
        for (int e = 0; e < 4; ++e) r.w[p][e] = pw[e];
      }
      // group entry: groups of <= 128 codes advance by 128 / g per chunk; 256 from the flat index
      const int64_t go = gs_log2 <= 7 ? (int64_t)(128 >> gs_log2) * ci
                                      : ((f_first[p] + 128 * ci) >> gs_log2) - (f_first[p] >> gs_log2);
      if (gs_log2 == 4) {  // groups of 16: the lane's two groups (the first even) in one dword
        r.dm[p] = *reinterpret_cast<const unsigned*>(pd[p] + go);
        r.zm[p] = *reinterpret_cast<const unsigned*>(pz[p] + go);
      } else {  // one group: its entry in the low half
        r.dm[p] = __half_as_ushort(pd[p][go]);
        r.zm[p] = __half_as_ushort(pz[p][go]);
      }
    }
  };
  // A operand of one chunk: the four 16-byte pieces x[m][128 c + 32 h + 8 s .. +7]
  auto load_x = [&](int i, u32x4 (&a)[4]) {
    const int ci = EXACT ? i : max(0, min(i, nrun - 1));
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const u32x4*>(xrow + 128 * ci + 8 * s);
  };
  // W_hat of one strip's 32 codes: o[s] is the B operand of k-step s (codes 8s .. 8s + 7)
  auto decode = [&](const WRegs& r, int p, u32x4 (&o)[4]) {
    const f16x2 dp = as_h2(r.dm[p]), zp = as_h2(r.zm[p]);
    float d[2], zd[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool e = gs_log2 == 4 && hh;  // groups of 16: the second half's own group
      const float dv = r.valid ? (float)(e ? dp[1] : dp[0]) : 0.f;
      const float zv = (float)(e ? zp[1] : zp[0]);
      d[hh] = dv;
      zd[hh] = r.valid ? zv * dv : 0.f;
    }
    if constexpr (FMT == 4) {
#pragma unroll
      for (int s = 0; s < 4; ++s) o[s] = wq8(r.w[p][s], d[s >> 1] * 16777216.0f, d[s >> 1] * 1048576.0f, zd[s >> 1]);
    } else if constexpr (FMT == 2) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float ds[4] = {d[hh] * 16777216.0f, d[hh] * 4194304.0f, d[hh] * 1048576.0f, d[hh] * 262144.0f};
        wq16_2b(r.w[p][hh], ds, zd[hh], o[2 * hh], o[2 * hh + 1]);
      }
    } else {
      decode32_3b(r.w[p], r.ph[p], d, zd, o);
    }
  };

  // The activations of a chunk are requested together with its codes: a wave's memory counter
  // completes in issue order, so a load issued later than the codes of a chunk further ahead
  // would make its wait cover those codes too.
  f32x4 acc[SP];
#pragma unroll
  for (int p = 0; p < SP; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  WRegs wr[RING];
  u32x4 xa[RING][4];
#pragma unroll
  for (int i = 0; i < (kDqAhead < NCW ? kDqAhead : NCW); ++i) {
    load_w(i, wr[i % RING]);
    load_x(i, xa[i % RING]);
  }
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    if (i + kDqAhead < NCW) {  // into the slot of chunk i - 1
      load_w(i + kDqAhead, wr[(i + kDqAhead) % RING]);
      load_x(i + kDqAhead, xa[(i + kDqAhead) % RING]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < SP; ++p) {
      u32x4 o[4];
      decode(wr[i % RING], p, o);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, xa[i % RING][s]),
                                                        __builtin_bit_cast(f16x8, o[s]), acc[p], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- the waves' partial sums in wave order; result lane (g, n) holds batch rows 4g .. 4g + 3
#pragma unroll
  for (int p = 0; p < SP; ++p) red[(wave * SP + p) * 64 + lane] = acc[p];
  __syncthreads();
  if (tid < 64 * SP) {
    const int p = tid >> 6, l = tid & 63;
    f32x4 s = red[p * 64 + l];
    for (int w = 1; w < nw; ++w) s += red[(w * SP + p) * 64 + l];
    const int64_t n = r0 + 16 * p + (l & 15);
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 4 * (l >> 4) + r;
        if (m < batch) {
          if (out_dtype == HQQ_OUT_F16)
            store_y<HQQ_OUT_F16>(y, m * N + n, s[r]);
          else
            store_y<HQQ_OUT_F32>(y, m * N + n, s[r]);
        }
      }
    }
  }
}

// Compile-time chunk counts per wave; a wave's run is at most ceil(C / waves) chunks.  3-bit
// stops at 24 (its 32-chunk body is past what the compiler unrolls).
constexpr int kDqNcw[] = {1, 2, 4, 6, 8, 12, 16, 24, 32};
constexpr int dq_ncw_count(int fmt) { return fmt == 3 ? 8 : 9; }

// EXACT: the waves' runs are all `need` chunks long and `need` is one of the counts.
template <int FMT, bool EXACT, int I = 0>
hipError_t launch_dq_ncw(int need, dim3 grid, dim3 block, hipStream_t st, const uint8_t* packed, const __half* delta,
                         const __half* zero, int64_t N, int64_t K, int gl, const __half* x, int64_t batch, void* y,
                         int y_dtype) {
  if constexpr (I < dq_ncw_count(FMT)) {
    if (EXACT ? need == kDqNcw[I] : need <= kDqNcw[I]) {
      hipLaunchKernelGGL((k_gemv_dq<FMT, kDqNcw[I], EXACT>), grid, block, 0, st, packed, delta, zero, N, K, gl, x,
                         batch, y, y_dtype);
      return hipGetLastError();
    }
    return launch_dq_ncw<FMT, EXACT, I + 1>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y,
                                            y_dtype);
  } else {
    return hipErrorInvalidValue;
  }
}

// Waves per block.
int dq_waves(int64_t) { return kDqMaxWaves; }

}  // namespace

bool gemv_dq_supported(int64_t N, int64_t K, int nbits, int g, int64_t batch) {
  if (nbits < 2 || nbits > 4 || batch < 1 || batch > 16 || K % 128 != 0 || N < 1) return false;
  if (g != 16 && g != 32 && g != 64 && g != 128 && g != 256) return false;
  if (nbits == 2 && g != 16) return false;
  const int64_t need = (K / 128 + dq_waves(N) - 1) / dq_waves(N);
  return need <= kDqNcw[dq_ncw_count(nbits) - 1];
}

hipError_t launch_gemv_dq(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                          int nbits, int g, const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  int gl = 0;
  while ((1 << gl) < g) ++gl;
  const int nw = dq_waves(N);
  const int64_t C = K / 128;
  const int need = (int)((C + nw - 1) / nw);
  bool exact = C % nw == 0;
  if (exact) {
    exact = false;
    for (int i = 0; i < dq_ncw_count(nbits); ++i) exact = exact || kDqNcw[i] == need;
  }
  const dim3 grid((unsigned)((N + kDqRows - 1) / kDqRows)), block(64 * nw);
  if (nbits == 3)
    return exact ? launch_dq_ncw<3, true>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype)
                 : launch_dq_ncw<3, false>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype);
  if (nbits == 4)
    return exact ? launch_dq_ncw<4, true>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype)
                 : launch_dq_ncw<4, false>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype);
  if (nbits == 2)
    return exact ? launch_dq_ncw<2, true>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype)
                 : launch_dq_ncw<2, false>(need, grid, block, st, packed, delta, zero, N, K, gl, x, batch, y, y_dtype);
  return hipErrorInvalidValue;
}

}  // namespace hqq
