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

#include "hqq_internal.h"

namespace hqq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_h2(unsigned u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ unsigned as_u(f16x2 h) { return __builtin_bit_cast(unsigned, h); }

// Eight 4-bit codes -> exact fp16 in the order [c0, c4, 16c1, 16c5, c2, c6, 16c3, 16c7].
__device__ __forceinline__ void unpack8(unsigned d, f16x2 (&p)[4]) {
  const unsigned d8 = d >> 8;
  const f16x2 off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  p[0] = as_h2((d & 0x000F000Fu) | 0x64006400u) + off;
  p[1] = as_h2((d & 0x00F000F0u) | 0x64006400u) + off;
  p[2] = as_h2((d8 & 0x000F000Fu) | 0x64006400u) + off;
  p[3] = as_h2((d8 & 0x00F000F0u) | 0x64006400u) + off;
}

__device__ __forceinline__ f16x8 cat(const f16x2 (&p)[4]) {
  return f16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
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

// ------------------------------------------------------------------------------------------
// GEMV, batch B <= 8.  Block = 8 waves on one 16-row strip; wave w takes the 128-code chunks
// c = w, w + 8, ... of each K segment.  Per segment the activations are staged in LDS in the
// operand order (x, with 1/16 on odd codes) together with the per-group sums of x; the eight
// waves' partial results are added in a fixed order at the end.
// ------------------------------------------------------------------------------------------
template <int B>
struct GemvCfg {
  static constexpr int CPW = (B <= 2) ? 8 : (B <= 4 ? 4 : 2);  // chunks per wave per segment
  static constexpr int KS = 128 * 8 * CPW;                       // K per segment
};

template <int B, int GS, int OUT>
__global__ void __launch_bounds__(512) k_gemv(const uint8_t* __restrict__ packed, const __half* __restrict__ delta,
                                              const __half* __restrict__ zero, int64_t N, int64_t K,
                                              const __half* __restrict__ x, void* __restrict__ y) {
  constexpr int CPW = GemvCfg<B>::CPW, KS = GemvCfg<B>::KS;
  constexpr int GPS = KS / GS;  // groups per segment
  extern __shared__ float lds[];
  float* sx = lds;                                               // [B][GPS]
  float* red = sx + B * GPS;                                     // [8][B][16]
  _Float16* xs = reinterpret_cast<_Float16*>(red + 8 * B * 16);  // [B][KS]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 4, nl = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + nl;
  const int64_t gpr = K / GS;  // groups per row
  const uint8_t* wrow = packed + n * (K / 2);
  const __half* drow = delta + n * gpr;
  const __half* zrow = zero + n * gpr;
  const int qh = quarter_of(h);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t nchunks = K / 128;
  for (int64_t kbase = 0; kbase < K; kbase += KS) {
    const int64_t cbase = kbase / 128;
    // issue this wave's weight loads for the segment first
    uint4 v[CPW];
    unsigned dm[CPW], zm[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int64_t c = cbase + wave + 8 * i;
      if (c < nchunks) {
        v[i] = *reinterpret_cast<const uint4*>(wrow + c * 64 + h * 16);
        if constexpr (GS == 64) {
          dm[i] = *reinterpret_cast<const unsigned*>(drow + 2 * c);
          zm[i] = *reinterpret_cast<const unsigned*>(zrow + 2 * c);
        } else {
          dm[i] = __half_as_ushort(drow[c]);
          zm[i] = __half_as_ushort(zrow[c]);
        }
      }
    }
    // stage x for the segment: 8-element blocks, operand order, 1/16 on the odd codes
    const int64_t klen = (K - kbase < KS) ? (K - kbase) : KS;
    const int nb = (int)(klen / 8);
    for (int idx = tid; idx < B * (KS / 8); idx += 512) {
      const int m = idx / (KS / 8), kb = idx % (KS / 8);
      uint4 o = make_uint4(0, 0, 0, 0);
      float part = 0.f;
      if (kb < nb) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x + m * K + kbase + 8 * kb);
        const unsigned r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) part += (float)as_h2(r4[t])[0] + (float)as_h2(r4[t])[1];
        o = perm_slots(raw);
        const f16x2 sc = {(_Float16)1.0f, (_Float16)0.0625f};
        // pairs (x0,x4),(x2,x6) keep scale 1; (x1,x5),(x3,x7) get 1/16
        o.y = as_u(as_h2(o.y) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        o.w = as_u(as_h2(o.w) * f16x2{(_Float16)0.0625f, (_Float16)0.0625f});
        (void)sc;
      }
      *reinterpret_cast<uint4*>(xs + m * KS + 8 * kb) = o;
      // group sums of the unscaled x: GS/8 consecutive blocks belong to one group
      part = seg_sum_f<GS / 8>(part);
      if ((kb % (GS / 8)) == 0) sx[m * GPS + kb / (GS / 8)] = part;
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int64_t c = cbase + wave + 8 * i;
      if (c >= nchunks) break;
      const int cl = (int)(c - cbase);  // chunk within the segment
      if constexpr (GS == 64) {
        // regroup: lanes 0-31 get the other half's first quarter pair, lanes 32-63 ours
        const auto s0 = __builtin_amdgcn_permlane32_swap(v[i].x, v[i].z, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(v[i].y, v[i].w, false, false);
        const unsigned grp_d[2][2] = {{s0[0], s1[0]}, {s0[1], s1[1]}};
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            f16x2 p[4];
            unpack8(grp_d[gg][s], p);
            const int kl = cl * 128 + gg * 64 + qh * 16 + s * 8;
            f16x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
            if (nl < B) A = *reinterpret_cast<const f16x8*>(xs + nl * KS + kl);
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, cat(p), P, 0, 0, 0);
          }
          const float dl = __half2float(__ushort_as_half((unsigned short)(dm[i] >> (16 * gg))));
          const float zz = __half2float(__ushort_as_half((unsigned short)(zm[i] >> (16 * gg))));
          const int gl = cl * 2 + gg;
#pragma unroll
          for (int r = 0; r < (B < 4 ? B : 4); ++r) {
            const int m = 4 * h + r;
            const float sxv = (m < B) ? sx[m * GPS + gl] : 0.f;
            acc[r] = fmaf(dl, fmaf(-zz, sxv, P[r]), acc[r]);
          }
        }
      } else {  // GS == 128: the 128-code chunk is one group; lane group h holds codes 32h..32h+31
        const unsigned dd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          f16x2 p[4];
          unpack8(dd[s], p);
          const int kl = cl * 128 + h * 32 + s * 8;
          f16x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
          if (nl < B) A = *reinterpret_cast<const f16x8*>(xs + nl * KS + kl);
          P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, cat(p), P, 0, 0, 0);
        }
        const float dl = __half2float(__ushort_as_half((unsigned short)dm[i]));
        const float zz = __half2float(__ushort_as_half((unsigned short)zm[i]));
#pragma unroll
        for (int r = 0; r < (B < 4 ? B : 4); ++r) {
          const int m = 4 * h + r;
          const float sxv = (m < B) ? sx[m * GPS + cl] : 0.f;
          acc[r] = fmaf(dl, fmaf(-zz, sxv, P[r]), acc[r]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < (B < 4 ? B : 4); ++r) {
    const int m = 4 * h + r;
    if (m < B) red[(wave * B + m) * 16 + nl] = acc[r];
  }
  __syncthreads();
  if (tid < B * 16) {
    const int m = tid / 16, col = tid % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[(w * B + m) * 16 + col];
    store_y<OUT>(y, (int64_t)m * N + n0 + col, sum);
  }
}

// ------------------------------------------------------------------------------------------
// GEMM, batch > 8.  Block = 4 waves, tile 128 batch rows x 64 output rows; wave w owns the
// output rows n0 + 16w .. +15 and all eight 16-row batch tiles.  Per 128-code chunk the block
// stages x (operand order) in LDS; each wave unpacks and dequantises its own weight rows to
// fp16 W_hat directly in the B-operand layout.
// ------------------------------------------------------------------------------------------
constexpr int kGemmM = 128;
constexpr int kXRow = 128 + 8;  // LDS row stride (halves) of the x tile

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

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t nchunks = K / 128;
  uint4 vnext = *reinterpret_cast<const uint4*>(wrow + h * 16);
  for (int64_t c = 0; c < nchunks; ++c) {
    const uint4 v = vnext;
    if (c + 1 < nchunks) vnext = *reinterpret_cast<const uint4*>(wrow + (c + 1) * 64 + h * 16);
    // stage x[m0 .. m0+127][128c .. 128c+127]
    for (int idx = tid; idx < kGemmM * 16; idx += 256) {
      const int mr = idx >> 4, kb = idx & 15;
      uint4 o = make_uint4(0, 0, 0, 0);
      if (m0 + mr < batch) o = perm_slots(*reinterpret_cast<const uint4*>(x + (m0 + mr) * K + c * 128 + 8 * kb));
      *reinterpret_cast<uint4*>(xt + mr * kXRow + 8 * kb) = o;
    }
    // weights of this chunk -> fp16 W_hat in operand order, per 64-code group
    f16x8 Bop[4];
    int kofs[4];
    if constexpr (GS == 64) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
      const unsigned gd[4] = {s0[0], s1[0], s0[1], s1[1]};
      const unsigned dmw = *reinterpret_cast<const unsigned*>(drow + 2 * c);
      const unsigned zmw = *reinterpret_cast<const unsigned*>(zrow + 2 * c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gg = j >> 1, s = j & 1;
        const _Float16 dl = __builtin_bit_cast(_Float16, (unsigned short)(dmw >> (16 * gg)));
        const _Float16 zz = __builtin_bit_cast(_Float16, (unsigned short)(zmw >> (16 * gg)));
        const f16x2 z1 = {zz, zz}, d1 = {dl, dl};
        const f16x2 z16 = z1 * f16x2{(_Float16)16.0f, (_Float16)16.0f};
        const f16x2 d16 = d1 * f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
        f16x2 p[4];
        unpack8(gd[j], p);
        p[0] = (p[0] - z1) * d1;
        p[1] = (p[1] - z16) * d16;
        p[2] = (p[2] - z1) * d1;
        p[3] = (p[3] - z16) * d16;
        Bop[j] = cat(p);
        kofs[j] = gg * 64 + qh * 16 + s * 8;
      }
    } else {
      const unsigned dd[4] = {v.x, v.y, v.z, v.w};
      const _Float16 dl = __builtin_bit_cast(_Float16, __half_as_ushort(drow[c]));
      const _Float16 zz = __builtin_bit_cast(_Float16, __half_as_ushort(zrow[c]));
      const f16x2 z1 = {zz, zz}, d1 = {dl, dl};
      const f16x2 z16 = z1 * f16x2{(_Float16)16.0f, (_Float16)16.0f};
      const f16x2 d16 = d1 * f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x2 p[4];
        unpack8(dd[j], p);
        p[0] = (p[0] - z1) * d1;
        p[1] = (p[1] - z16) * d16;
        p[2] = (p[2] - z1) * d1;
        p[3] = (p[3] - z16) * d16;
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
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 16 * t + 4 * h + r;
      if (wvalid && m < batch) store_y<OUT>(y, m * N + n, acc[t][r]);
    }
}

template <int B, int GS>
hipError_t gemv_b(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                  const __half* x, void* y, int y_dtype, hipStream_t st) {
  const size_t lds = gemv_lds_bytes(K, GS, B);
  const dim3 grid((unsigned)(N / 16));
  if (y_dtype == HQQ_OUT_F16)
    hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F16>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
  else
    hipLaunchKernelGGL((k_gemv<B, GS, HQQ_OUT_F32>), grid, dim3(512), lds, st, packed, delta, zero, N, K, x, y);
  return hipGetLastError();
}

template <int GS>
hipError_t gemv_gs(const uint8_t* packed, const __half* delta, const __half* zero, int64_t N, int64_t K,
                   const __half* x, int64_t batch, void* y, int y_dtype, hipStream_t st) {
  switch (batch) {
    case 1: return gemv_b<1, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 2: return gemv_b<2, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 3: return gemv_b<3, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 4: return gemv_b<4, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 5: return gemv_b<5, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 6: return gemv_b<6, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 7: return gemv_b<7, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    case 8: return gemv_b<8, GS>(packed, delta, zero, N, K, x, y, y_dtype, st);
    default: return hipErrorInvalidValue;
  }
}

template <int B>
size_t gemv_lds_b(int64_t K, int gs) {
  (void)K;
  constexpr int KS = GemvCfg<B>::KS;
  return (size_t)B * (KS / gs) * 4 + (size_t)8 * B * 16 * 4 + (size_t)B * KS * 2;
}

}  // namespace

size_t gemv_lds_bytes(int64_t K, int gs, int64_t batch) {
  switch (batch) {
    case 1: return gemv_lds_b<1>(K, gs);
    case 2: return gemv_lds_b<2>(K, gs);
    case 3: return gemv_lds_b<3>(K, gs);
    case 4: return gemv_lds_b<4>(K, gs);
    case 5: return gemv_lds_b<5>(K, gs);
    case 6: return gemv_lds_b<6>(K, gs);
    case 7: return gemv_lds_b<7>(K, gs);
    case 8: return gemv_lds_b<8>(K, gs);
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
