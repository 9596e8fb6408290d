// HQQ quantizer kernels for gfx950 (CDNA4).
//
// Method (page "HQQ 算法解读", sections "第一拍", "第二拍", "为什么 zero 是这个均值",
// "shrink 不是删除极值", "axis 不是一个无关紧要的开关", "为什么一定要分组"):
//   per group: min-max start s = (2^b-1)/(max-min) (1 when the range is tiny, at most 2e4),
//   z0 = -min*s, delta = 1/s; then rounds k = 0..: q = clip(rint(W*s + z_k)), W_hat =
//   (q - z_k)*delta, r = W - W_hat, err_k = sum|r|, e = shrink(r; beta_k, p),
//   z_(k+1) = mean(q - (W - e)*s); the whole-tensor MAE of round k decides the stop;
//   final codes q = clip(rint(W*s + z_kept)).
//
// Mapping: a group of g weights is held by L lanes of one 64-wide wave, E = g/L weights per
// lane in VGPRs (fp64 W and W*s, both formed once), so the whole iteration runs out of
// registers.  Group sums (|r| and the zero update) and the min/max start are reduced over
// the L lanes with DPP row permutations (quad_perm, row_half_mirror, row_mirror), which give
// every lane of the group the bit-identical result.  All solver arithmetic is fp64 with no
// contraction (the library is built with -ffp-contract=off), in the operation order of the
// method; only the summation order inside a group differs from a sequential sum.
//
// Global early stop without host round trips: each block writes, per round, the sum of its
// groups' |r| sums (fixed order) to the workspace; a one-block kernel adds the block sums in
// a fixed order, forms MAE_k, applies the stop rule and stores the index of the kept zero
// on the device.  The solve pass speculates that the loop runs all rounds and writes the
// final codes for z_iters directly; a fix-up pass (same kernel, reading the index from
// device memory) redoes the groups only when the loop stopped early.
//
// Frozen groups: when a round leaves the zero unchanged (z_(k+1) == z_k bit for bit) and
// every residual is below the smallest shrink threshold of the remaining rounds, every later
// round repeats this one exactly (same q, same r, e = 0, same zero), so the wave stops
// computing once all its groups are frozen and fills the remaining rounds' |r| sums with the
// last value.  The results are identical to running every round.
//
// Shrink fast path: e = 0 exactly when |r| <= beta^(-1/(2-p)); the kernel takes e = 0 for
// |r| below that threshold times (1 - 1e-6) (a margin far above the rounding of the
// expression) and evaluates the shrink with pow() otherwise.  Both this and the freeze test
// look at each lane's sum of |r|, an upper bound of every |r| of the lane.

#include "hqq_internal.h"

namespace hqq {
namespace {

// ------------------------------------------------------------------------------------------
// Cross-lane reductions inside aligned segments of L lanes (L in 1, 2, 4, 8, 16), by DPP.
// ------------------------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

// Every control used here names a valid source lane for every lane and all rows and banks are
// enabled, so no lane keeps its old value: a plain DPP move of the two halves (no register
// to pre-fill, unlike an update with an old operand).
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int L>
__device__ __forceinline__ double seg_sum(double v) {
  if constexpr (L >= 2) v = v + dpp<kDppXor1>(v);
  if constexpr (L >= 4) v = v + dpp<kDppXor2>(v);
  if constexpr (L >= 8) v = v + dpp<kDppHalfMirror>(v);
  if constexpr (L >= 16) v = v + dpp<kDppMirror>(v);
  return v;
}
template <int L>
__device__ __forceinline__ double seg_min(double v) {
  if constexpr (L >= 2) v = fmin(v, dpp<kDppXor1>(v));
  if constexpr (L >= 4) v = fmin(v, dpp<kDppXor2>(v));
  if constexpr (L >= 8) v = fmin(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = fmin(v, dpp<kDppMirror>(v));
  return v;
}
template <int L>
__device__ __forceinline__ double seg_max(double v) {
  if constexpr (L >= 2) v = fmax(v, dpp<kDppXor1>(v));
  if constexpr (L >= 4) v = fmax(v, dpp<kDppXor2>(v));
  if constexpr (L >= 8) v = fmax(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = fmax(v, dpp<kDppMirror>(v));
  return v;
}

// Balanced pairwise sum of v[LO .. LO+N) (N a power of two), left half + right half.  With the
// lane-level DPP tree below this makes every group sum the balanced pairwise sum in index
// order over the whole group, the summation order fixed for every sum of the method.
template <int LO, int N, int E>
__device__ __forceinline__ double tree_sum(const double (&v)[E]) {
  if constexpr (N == 1)
    return v[LO];
  else
    return tree_sum<LO, N / 2, E>(v) + tree_sum<LO + N / 2, N / 2, E>(v);
}

// fp64 -> fp16 bits, round to nearest even: round to odd into fp32 (24 >= 11 + 2 bits, so the
// second rounding is exact), then the hardware fp32 -> fp16 conversion.
__device__ __forceinline__ unsigned short f64_to_f16_bits(double x) {
  const float f = (float)x;
  unsigned u = __float_as_uint(f);
  const double back = (double)f;
  if (back != x && !__builtin_isinf(f)) {
    if (fabs(back) > fabs(x)) u -= 1u;
    u |= 1u;
  }
  return __half_as_ushort(__float2half_rn(__uint_as_float(u)));
}

__device__ __forceinline__ void store_meta(void* p, int dtype, int64_t j, double v) {
  if (dtype == HQQ_META_F16)
    reinterpret_cast<unsigned short*>(p)[j] = f64_to_f16_bits(v);
  else if (dtype == HQQ_META_F32)
    reinterpret_cast<float*>(p)[j] = (float)v;
  else
    reinterpret_cast<double*>(p)[j] = v;
}

// |r| - |r|^(p-1)/beta for the shrink's rare slow path; kept out of line so that pow's
// temporaries do not raise the register count of the whole solver.
__device__ __noinline__ double shrink_mag(double a, double pm1, double beta) { return a - pow(a, pm1) / beta; }

// Lanes per group (L) and weights per lane (E) for a group size.
template <int G>
struct Shape {
  static constexpr int E = (G == 16) ? 4 : (G >= 256 ? 16 : 8);
  static constexpr int L = G / E;
  static constexpr int GPW = 64 / L;  // groups per wave
  static_assert(L >= 1 && L <= 16 && E * L == G, "group size");
};

// Waves per SIMD the solve kernels are compiled for (the register budget is 512 / waves).
// The solver is bound by fp64 latency rather than issue, so more resident waves pay: g <= 128
// fits 4 (5 at g = 16); g = 256 (16 weights per lane) keeps its natural 2.  On axis 1 this
// costs no spill; on axis 0 some ten registers of per-tile addresses spill outside the round
// loop.  One wave more than that (5, or 6 at g = 16) spills inside the round loop and halves
// the speed.
template <int G>
constexpr int solve_waves() { return G == 16 ? 5 : (G >= 256 ? 2 : 4); }

// ------------------------------------------------------------------------------------------
// One proximal round of one group (per lane: E weights).  Returns the group's sum of |r|,
// the next zero and a bound on this lane's largest |r|: the lane's own pairwise sum of |r|
// (a rounded sum of non-negative terms is at least each term), which the shrink and freeze
// tests use in place of the maximum (both stay sufficient; the maximum would cost an
// instruction per weight and round).
// ------------------------------------------------------------------------------------------
template <int E, int L>
__device__ __forceinline__ void hqq_round(const double (&w)[E], const double (&ws)[E], double s, double delta,
                                          double z, double qmax, double beta, double pm1, double thr,
                                          double inv_g, double sws, double& err_o, double& zn_o, double& maxr_o) {
  double ar[E], qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double t = ws[e] + z;
    double qq = __builtin_rint(t);
    qq = fmax(qq, 0.0);
    qq = fmin(qq, qmax);
    const double rr = __builtin_fma(-(qq - z), delta, w[e]);  // W - (q - z) delta, one rounding
    ar[e] = fabs(rr);
    qv[e] = qq;
  }
  const double err = tree_sum<0, E, E>(ar);
  double su = sws;  // the group's sum of (W - e) s: sum W s while the shrink is zero
  if (__any(err >= thr)) {
    // Some residual of the wave may pass the shrink: redo the terms with the shrink evaluated
    // wherever it can be non-zero (q and r recomputed identically).
    double u[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double t = ws[e] + z;
      double qq = __builtin_rint(t);
      qq = fmax(qq, 0.0);
      qq = fmin(qq, qmax);
      const double rr = __builtin_fma(-(qq - z), delta, w[e]);
      const double a = fabs(rr);
      double ee = 0.0;
      if (a >= thr) {
        const double v = shrink_mag(a, pm1, beta);
        if (v > 0.0) ee = (rr < 0.0) ? -v : v;
      }
      u[e] = (ee == 0.0) ? ws[e] : (w[e] - ee) * s;
    }
    su = seg_sum<L>(tree_sum<0, E, E>(u));
  }
  // the codes are integers: their sum is exact in any order
  const double sq = seg_sum<L>(tree_sum<0, E, E>(qv));
  err_o = seg_sum<L>(err);
  zn_o = (sq - su) * inv_g;
  maxr_o = err;
}

// Start of a group from its weights (min-max), then the rounds.  Returns the final zero.
// err_lds (nullptr in the fix-up pass) receives the group's |r| sum per round at
// err_lds[k * stride]; rounds after the wave froze get the frozen value.
template <int E, int L>
__device__ __forceinline__ double solve_group(const SolveArgs& a, const double (&w)[E], double (&ws)[E],
                                              bool valid, int kmax, double* err_lds, int stride, bool write_err,
                                              double& s_o, double& delta_o, int& kfrozen) {
  double mn = w[0], mx = w[0];
#pragma unroll
  for (int e = 1; e < E; ++e) {
    mn = fmin(mn, w[e]);
    mx = fmax(mx, w[e]);
  }
  mn = seg_min<L>(mn);
  mx = seg_max<L>(mx);
  const double d = mx - mn;
  double s = (d <= a.tiny) ? 1.0 : a.qmax / d;
  s = fmin(s, HQQ_MAX_SCALE);
  const double delta = 1.0 / s;
  double z = -mn * s;
#pragma unroll
  for (int e = 0; e < E; ++e) ws[e] = w[e] * s;
  const double sws = seg_sum<L>(tree_sum<0, E, E>(ws));  // the group's sum of W s (pairwise)

  const double inv_g = 1.0 / (double)(E * L);
  // canonicalised once here, not in every round's clip
  const double qmax = __builtin_canonicalize(a.qmax);
  kfrozen = kmax;  // the round at which every group of the wave froze (kmax: not before the end)
  double* slot = err_lds;  // round k's entry; the fill below continues from the same pointer
  // each round's two thresholds are requested a round ahead: a scalar load waited for at its
  // use would sit in the middle of every round
  double thr_k = a.thr[0], thf_k = a.thr_frozen[0];
  for (int k = 0; k < kmax; ++k) {
    const int kn = k + 1 < kmax ? k + 1 : k;
    const double thr_n = a.thr[kn], thf_n = a.thr_frozen[kn];
    double err, zn, maxr;
    hqq_round<E, L>(w, ws, s, delta, z, qmax, a.beta[k], a.pm1, thr_k, inv_g, sws, err, zn, maxr);
    const double ev = valid ? err : 0.0;
    if (write_err) *slot = ev;
    slot += stride;
    const bool frozen = !valid || (zn == z && maxr <= thf_k);
    thr_k = thr_n;
    thf_k = thf_n;
    z = zn;
    if (__all(frozen)) {
      if (write_err)
        for (int kk = k + 1; kk < a.iters; ++kk, slot += stride) *slot = ev;
      kfrozen = k;
      break;
    }
  }
  s_o = s;
  delta_o = delta;
  return z;
}

template <int E>
__device__ __forceinline__ void final_codes(const double (&ws)[E], double z, double qmax, unsigned (&c)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    double qq = __builtin_rint(ws[e] + z);
    qq = fmax(qq, 0.0);
    qq = fmin(qq, qmax);
    c[e] = (unsigned)qq;
  }
}

// The thread index through an empty asm statement: what is formed from it here is computed at
// this point, not hoisted above the round loop where it would only hold registers.
__device__ __forceinline__ int late_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Sum of the two 16-lane rows of each 32-lane half (SWAP16 = true) or of the two 32-lane halves
// of the wave, in every lane.  A swap of a register with itself gives the even (lower) and the
// odd (upper) part broadcast over both, so their sum is left + right with no lane index.
template <bool SWAP16>
__device__ __forceinline__ double add_across(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned l = (unsigned)b, h = (unsigned)(b >> 32);
  unsigned l0, l1, h0, h1;
  if constexpr (SWAP16) {
    const auto ls = __builtin_amdgcn_permlane16_swap(l, l, false, false);
    const auto hs = __builtin_amdgcn_permlane16_swap(h, h, false, false);
    l0 = ls[0]; l1 = ls[1]; h0 = hs[0]; h1 = hs[1];
  } else {
    const auto ls = __builtin_amdgcn_permlane32_swap(l, l, false, false);
    const auto hs = __builtin_amdgcn_permlane32_swap(h, h, false, false);
    l0 = ls[0]; l1 = ls[1]; h0 = hs[0]; h1 = hs[1];
  }
  return __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0)) +
         __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
}

// Sum of the per-group round errors of the block (pairwise, in group order) to the
// workspace, block-major [nblocks][iters].  One wave takes 64 / NG rounds at a time, lane
// NG r + i holding group i of its round r: DPP steps inside rows of 16 lanes, then the sums of
// row pairs and of wave halves (add_across).  After every step each lane of an aligned run holds that run's
// sum (the adds are commutative), so this is the balanced pairwise tree over the NG groups;
// no barrier after the first (a former LDS tree took one per level and an integer division
// per element).
template <int NG>
__device__ __forceinline__ void write_partials(const SolveArgs& a, const double* err_lds, int64_t tile) {
  static_assert(NG == 16 || NG == 32 || NG == 64, "groups per block");
  constexpr int RPW = 64 / NG;  // rounds per wave and pass
  __syncthreads();
  const int t = late_tid();
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nw = blockDim.x >> 6, r = lane / NG, i = lane % NG;
  for (int k0 = wave * RPW; k0 < a.iters; k0 += nw * RPW) {
    const int k = k0 + r;
    double v = (k < a.iters) ? err_lds[k * NG + i] : 0.0;
    v = seg_sum<16>(v);
    if constexpr (NG >= 32) v = add_across<true>(v);
    if constexpr (NG >= 64) v = add_across<false>(v);
    if (i == 0 && k < a.iters) a.partials[tile * a.iters + k] = v;
  }
}


// Wave 0 stores the steps and wave 1 the zeros (ng <= 64 groups per block), so the choice of
// array is uniform per wave.
__device__ __forceinline__ void store_block_meta(const SolveArgs& a, const double* meta_lds, int ng, int64_t g0) {
  __syncthreads();
  const int t = late_tid();
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  if (wave < 2 && lane < ng && g0 + lane < a.G)
    store_meta(wave == 0 ? a.delta : a.zero, a.meta_dtype, g0 + lane, meta_lds[wave * ng + lane]);
}

// 3-bit codes of one axis-1 tile (flat codes [T0, T1), T1 = T0 + TC or the tensor's end) from
// LDS, ten per 32-bit word at bits 3t: the words inside the tile are stored directly; the word
// the tile starts inside (T0 not a multiple of 10) and the word it ends inside get only this
// tile's codes, kept in a.edges3[2 tile] and [2 tile + 1] for k_merge3 (the tensor's last word,
// padded with code 0, is whole).
template <int TC>
__device__ __forceinline__ void pack3_tile(const SolveArgs& a, const uint8_t* ct, int64_t tile, int64_t N) {
  const int64_t T0 = tile * TC;
  const int64_t T1 = T0 + TC < N ? T0 + TC : N;  // T1 - T0 >= 16: a tile holds at least one group
  uint32_t* out = reinterpret_cast<uint32_t*>(a.packed);
  // every word holding a code of the tile, one per thread: whole words (and the tensor's padded
  // last word) to the output, the word the tile starts inside and the one it ends inside to edges3
  for (int64_t j = T0 / 10 + late_tid(); j <= (T1 - 1) / 10; j += blockDim.x) {
    const int64_t lo = 10 * j > T0 ? 10 * j : T0, hi = 10 * j + 10 < T1 ? 10 * j + 10 : T1;
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      const int64_t i = 10 * j + t;
      const bool in = i >= lo && i < hi;
      const uint32_t c = ct[in ? i - T0 : 0];
      w |= in ? c << (3 * t) : 0u;
    }
    if (lo > 10 * j)
      a.edges3[2 * tile] = w;
    else if (hi < 10 * j + 10 && T1 < N)
      a.edges3[2 * tile + 1] = w;
    else
      out[j] = w;
  }
}

// Whether the solve records, per tile, the round by which all its waves froze, so that the
// fix-up can skip tiles that an early stop does not change.  Only for 2-bit codes: their groups
// converge within a few rounds and the loop stops early, which makes the fix-up redo every
// group; at 3 and 4 bits the loop usually runs to the end, and the recording cost the solve 9 %
// (a different schedule of its round loop), so those widths keep the plain fix-up.
template <int NBITS>
constexpr bool kRecordFreeze = (NBITS == 2);

// ------------------------------------------------------------------------------------------
// axis = 1: group j = 64-bit-aligned run of g consecutive weights.  Block = 4 waves.
// ------------------------------------------------------------------------------------------
template <int NBITS, int G, bool FIX>
__device__ __forceinline__ void ax1_tile(const SolveArgs& a, int64_t tile, int kmax, double* err_lds,
                                         double* meta_lds) {
  using S = Shape<G>;
  constexpr int E = S::E, L = S::L, GPW = S::GPW;
  constexpr int GPB = 4 * GPW;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / L, slot = lane % L;
  const int gblock = wave * GPW + sub;
  const int64_t gidx = tile * GPB + gblock;
  const bool valid = gidx < a.G;
  const int64_t e0 = (valid ? gidx : 0) * G + slot * E;

  double w[E], ws[E];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.W + e0);
    if constexpr (E == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(a.W + e0);
      const unsigned u[2] = {v.x, v.y};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (double)__half2float(__ushort_as_half((unsigned short)(u[e >> 1] >> (16 * (e & 1)))));
    } else {
#pragma unroll
      for (int c = 0; c < E / 8; ++c) {
        const uint4 v = src[c];
        const unsigned u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w[8 * c + e] = (double)__half2float(__ushort_as_half((unsigned short)(u[e >> 1] >> (16 * (e & 1)))));
      }
    }
    if (!valid)
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] = 0.0;
  }

  double s, delta;
  int kfrozen;
  const double z =
      solve_group<E, L>(a, w, ws, valid, kmax, err_lds + gblock, GPB, !FIX && slot == 0, s, delta, kfrozen);
  __shared__ int s_kfrozen[4];
  if (kRecordFreeze<NBITS> && !FIX && lane == 0) s_kfrozen[wave] = kfrozen;  // published by store_block_meta

  unsigned c[E];
  final_codes<E>(ws, z, a.qmax, c);
  if (valid) {
    if constexpr (NBITS == 4) {
      if constexpr (E == 4) {
        reinterpret_cast<unsigned short*>(a.packed)[e0 / 4] =
            (unsigned short)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12));
      } else {
#pragma unroll
        for (int h = 0; h < E / 8; ++h) {
          unsigned word = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) word |= c[8 * h + e] << (4 * e);
          reinterpret_cast<unsigned*>(a.packed)[e0 / 8 + h] = word;
        }
      }
    } else if constexpr (NBITS == 2) {
      if constexpr (E == 4) {
        a.packed[e0 / 4] = (uint8_t)(c[0] | (c[1] << 2) | (c[2] << 4) | (c[3] << 6));
      } else {
#pragma unroll
        for (int h = 0; h < E / 8; ++h) {
          unsigned v = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) v |= c[8 * h + e] << (2 * e);
          reinterpret_cast<unsigned short*>(a.packed)[e0 / 8 + h] = (unsigned short)v;
        }
      }
    }
    if (slot == 0) {
      meta_lds[gblock] = delta;
      meta_lds[GPB + gblock] = z;
    }
  }
  uint8_t* ct = reinterpret_cast<uint8_t*>(meta_lds + 2 * GPB);  // 3-bit: the tile's codes, one byte each
  if constexpr (NBITS == 3) {
    const int o = gblock * G + slot * E;  // codes of groups past the tensor's end are never read
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<unsigned*>(ct + o + e) = c[e] | (c[e + 1] << 8) | (c[e + 2] << 16) | (c[e + 3] << 24);
  }
  store_block_meta(a, meta_lds, GPB, tile * GPB);  // its barrier also publishes the code tile
  if constexpr (NBITS == 3) pack3_tile<GPB * G>(a, ct, tile, a.G * (int64_t)G);
  if (kRecordFreeze<NBITS> && !FIX && threadIdx.x == 0)
    a.tile_round[tile] = max(max(s_kfrozen[0], s_kfrozen[1]), max(s_kfrozen[2], s_kfrozen[3]));
  if (!FIX) write_partials<GPB>(a, err_lds, tile);
}

template <int NBITS, int G, bool FIX>
__global__ void __launch_bounds__(256, solve_waves<G>()) k_quant_ax1(const SolveArgs a) {
  extern __shared__ double err_lds[];  // [iters][groups per block], then [2][groups per block]
  constexpr int GPB = 4 * Shape<G>::GPW;
  double* meta_lds = err_lds + a.iters * GPB;
  int kmax = a.iters;
  if (FIX) {
    kmax = a.ctrl[0];
    if (kmax >= a.iters) return;  // the loop ran to the end: the solve pass wrote the result
  }
  for (int64_t tile = blockIdx.x; tile < a.nblocks; tile += gridDim.x) {
    // fix-up: every wave of this tile froze by round kmax, after which its zeros no longer
    // change, so the solve pass already wrote the codes and zeros of z_kmax
    if (kRecordFreeze<NBITS> && FIX && a.tile_round[tile] <= kmax) continue;
    ax1_tile<NBITS, G, FIX>(a, tile, kmax, err_lds, meta_lds);
    if (FIX) __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// Scale search (the second, slower solver the method names: it can grid-search the scale while
// the default keeps the min-max scale).  Reading: per group and multiplier c_j of the grid,
// s = min(s0 c_j, 2e4) with s0 the min-max start before its limit, delta = 1/s, z0 = -min s,
// the proximal rounds with the stop rule applied to the group's own error sum (keep z_(k-1) at
// the first k >= 1 whose sum is not below the previous one, else z_iters), and the error sum of
// the candidate's final codes; candidate 0 first, a later one only with a strictly smaller
// error.  One tile of 4 GPW groups per block as in the solve pass (axis 0: a column tile staged
// through LDS); a wave runs the rounds of a candidate until every one of its groups has
// stopped.  No global dependency (the 3-bit codes go through a byte per code and k_pack3, as in
// the default path).
// ------------------------------------------------------------------------------------------
// The search for one group from a lane's E weights (L lanes per group): the chosen scale, step,
// zero and index.  Every lane of the group ends with the same values (the DPP sums and maxima
// give each lane the bit-identical result).
template <int E, int L>
__device__ __forceinline__ void v2_search(const SolveArgs& a, const ScaleGrid& sg, const double (&w)[E], bool valid,
                                          double& best_s, double& best_delta, double& best_z, int& best_c) {
  double mn = w[0], mx = w[0];
#pragma unroll
  for (int e = 1; e < E; ++e) {
    mn = fmin(mn, w[e]);
    mx = fmax(mx, w[e]);
  }
  mn = seg_min<L>(mn);
  mx = seg_max<L>(mx);
  const double d = mx - mn;
  const double sb = (d <= a.tiny) ? 1.0 : a.qmax / d;
  const double qmax = __builtin_canonicalize(a.qmax);
  const double inv_g = 1.0 / (double)(E * L);

  double best_e = 0.0;
  best_s = best_delta = best_z = 0.0;
  best_c = 0;
  double ws[E];
  for (int c = 0; c < sg.n; ++c) {
    const double s = fmin(sb * sg.c[c], HQQ_MAX_SCALE);
    const double delta = 1.0 / s;
    double z = -mn * s;
#pragma unroll
    for (int e = 0; e < E; ++e) ws[e] = w[e] * s;
    const double sws = seg_sum<L>(tree_sum<0, E, E>(ws));  // the group's sum of W s (pairwise)
    double zprev = z, best = __builtin_inf();
    bool done = !valid;
    double thr_k = a.thr[0];  // requested a round ahead, as in the solve
    for (int k = 0; k < a.iters; ++k) {
      if (__all(done)) break;
      const double thr_n = a.thr[k + 1 < a.iters ? k + 1 : k];
      double err, zn, bound;
      hqq_round<E, L>(w, ws, s, delta, z, qmax, a.beta[k], a.pm1, thr_k, inv_g, sws, err, zn, bound);
      thr_k = thr_n;
      if (!done) {
        if (k >= 1 && !(err < best)) {
          z = zprev;
          done = true;
        } else {
          best = err;
          zprev = z;
          z = zn;
        }
      }
    }
    double ar[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      double qq = __builtin_rint(ws[e] + z);
      qq = fmax(qq, 0.0);
      qq = fmin(qq, qmax);
      ar[e] = fabs(w[e] - (qq - z) * delta);
    }
    const double ce = seg_sum<L>(tree_sum<0, E, E>(ar));
    if (c == 0 || ce < best_e) {
      best_e = ce;
      best_s = s;
      best_delta = delta;
      best_z = z;
      best_c = c;
    }
  }
}

template <int NBITS, int G>
__global__ void __launch_bounds__(256) k_quant_v2(const SolveArgs a, const ScaleGrid sg) {
  using S = Shape<G>;
  constexpr int E = S::E, L = S::L, GPW = S::GPW;
  constexpr int GPB = 4 * GPW;
  extern __shared__ double meta_lds[];  // [2][groups per block]
  const int64_t tile = blockIdx.x;
  if (tile >= a.nblocks) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / L, slot = lane % L;
  const int gblock = wave * GPW + sub;
  const int64_t gidx = tile * GPB + gblock;
  const bool valid = gidx < a.G;
  const int64_t e0 = (valid ? gidx : 0) * G + slot * E;

  double w[E];
#pragma unroll
  for (int c = 0; c < E / 2; ++c) {
    const unsigned u = reinterpret_cast<const unsigned*>(a.W + e0)[c];
    w[2 * c] = valid ? (double)__half2float(__ushort_as_half((unsigned short)(u & 0xFFFFu))) : 0.0;
    w[2 * c + 1] = valid ? (double)__half2float(__ushort_as_half((unsigned short)(u >> 16))) : 0.0;
  }
  double best_s, best_delta, best_z;
  int best_c;
  v2_search<E, L>(a, sg, w, valid, best_s, best_delta, best_z, best_c);

  double ws[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ws[e] = w[e] * best_s;
  unsigned cq[E];
  final_codes<E>(ws, best_z, __builtin_canonicalize(a.qmax), cq);
  if (valid) {
    if constexpr (NBITS == 4) {
      if constexpr (E == 4) {
        reinterpret_cast<unsigned short*>(a.packed)[e0 / 4] =
            (unsigned short)(cq[0] | (cq[1] << 4) | (cq[2] << 8) | (cq[3] << 12));
      } else {
#pragma unroll
        for (int h = 0; h < E / 8; ++h) {
          unsigned word = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) word |= cq[8 * h + e] << (4 * e);
          reinterpret_cast<unsigned*>(a.packed)[e0 / 8 + h] = word;
        }
      }
    } else if constexpr (NBITS == 2) {
      if constexpr (E == 4) {
        a.packed[e0 / 4] = (uint8_t)(cq[0] | (cq[1] << 2) | (cq[2] << 4) | (cq[3] << 6));
      } else {
#pragma unroll
        for (int h = 0; h < E / 8; ++h) {
          unsigned v = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) v |= cq[8 * h + e] << (2 * e);
          reinterpret_cast<unsigned short*>(a.packed)[e0 / 8 + h] = (unsigned short)v;
        }
      }
    } else {  // 3-bit: one byte per code, packed by k_pack3
#pragma unroll
      for (int h = 0; h < E / 4; ++h)
        reinterpret_cast<unsigned*>(a.codes_ws + e0)[h] =
            cq[4 * h] | (cq[4 * h + 1] << 8) | (cq[4 * h + 2] << 16) | (cq[4 * h + 3] << 24);
    }
    if (slot == 0) {
      meta_lds[gblock] = best_delta;
      meta_lds[GPB + gblock] = best_z;
      if (sg.choice) sg.choice[gidx] = (uint8_t)best_c;
    }
  }
  store_block_meta(a, meta_lds, GPB, tile * GPB);
}

// Axis 0: the block stages its g x TW column tile through LDS as the axis-0 solve does, each
// lane takes E weights of one column, the search runs as on axis 1, and the codes go back
// through LDS for row-wise packed stores.
// Tile of the axis-0 grid's t-th block: blocks run round-robin over the 8 XCDs (block t on XCD
// t mod 8), and a tile's rows are TW columns of the [g, M] view, a few bytes of each of g rows
// M apart, so the tiles that share a cache line must run on one XCD's L2: XCD x takes the x-th
// eighth of the tiles in order (a bijection; the last nblocks mod 8 tiles keep their index).
// In order, each L2 line of the weights is fetched once and each line of codes written back
// once (measured 4.0x the weight and code bytes with consecutive tiles on different XCDs).
__device__ __forceinline__ int64_t ax0_tile_of(int64_t t, int64_t nblocks) {
  const int64_t full = nblocks & ~int64_t(7);
  return t < full ? (t & 7) * (full >> 3) + (t >> 3) : t;
}

template <int NBITS, int G>
__global__ void __launch_bounds__(256) k_quant_v2_ax0(const SolveArgs a, const ScaleGrid sg) {
  using S = Shape<G>;
  constexpr int E = S::E, L = S::L, GPW = S::GPW;
  constexpr int TW = 4 * GPW;  // groups per block, as in the axis-0 solve
  constexpr int CPR = TW / 8, ROW = TW + 8, NT = 256;
  extern __shared__ double smem[];
  double* meta_lds = smem;                                   // [2][TW]
  __half* wt = reinterpret_cast<__half*>(smem + 2 * TW);     // [G][ROW]
  uint8_t* ct = reinterpret_cast<uint8_t*>(wt);              // [G][TW] after the loads
  if (blockIdx.x >= a.nblocks) return;
  const int64_t tile = ax0_tile_of(blockIdx.x, a.nblocks);
  const int64_t M = a.G, j0 = tile * TW;
  const int tid = threadIdx.x;
  for (int task = tid; task < G * CPR; task += NT) {
    const int i = task / CPR, c = task % CPR;
    const int64_t col = j0 + 8 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < M) v = *reinterpret_cast<const uint4*>(a.W + (int64_t)i * M + col);
    *reinterpret_cast<uint4*>(wt + i * ROW + 8 * c) = v;
  }
  __syncthreads();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane % L, acol = wave * GPW + lane / L;
  const int64_t gidx = j0 + acol;
  const bool valid = gidx < M;
  double w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = valid ? (double)__half2float(wt[(slot * E + e) * ROW + acol]) : 0.0;
  __syncthreads();  // the tile is reused for the codes below

  double best_s, best_delta, best_z;
  int best_c;
  v2_search<E, L>(a, sg, w, valid, best_s, best_delta, best_z, best_c);

  double ws[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ws[e] = w[e] * best_s;
  unsigned cq[E];
  final_codes<E>(ws, best_z, __builtin_canonicalize(a.qmax), cq);
#pragma unroll
  for (int e = 0; e < E; ++e) ct[(slot * E + e) * TW + acol] = (uint8_t)cq[e];
  if (valid && slot == 0) {
    meta_lds[acol] = best_delta;
    meta_lds[TW + acol] = best_z;
    if (sg.choice) sg.choice[gidx] = (uint8_t)best_c;
  }
  store_block_meta(a, meta_lds, TW, j0);  // its barrier also publishes the code tile
  for (int task = tid; task < G * CPR; task += NT) {  // rows of TW codes, 8 per task
    const int i = task / CPR, cc = task % CPR;
    if (j0 + 8 * cc >= M) continue;
    const uint8_t* cr = ct + i * TW + 8 * cc;
    const int64_t f = (int64_t)i * M + j0 + 8 * cc;
    if constexpr (NBITS == 4) {
      unsigned word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= (unsigned)cr[e] << (4 * e);
      reinterpret_cast<unsigned*>(a.packed)[f / 8] = word;
    } else if constexpr (NBITS == 2) {
      unsigned v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (unsigned)cr[e] << (2 * e);
      reinterpret_cast<unsigned short*>(a.packed)[f / 8] = (unsigned short)v;
    } else {
      *reinterpret_cast<uint2*>(a.codes_ws + f) = *reinterpret_cast<const uint2*>(cr);
    }
  }
}

// ------------------------------------------------------------------------------------------
// axis = 0: group j = {i*M + j}, a column of the [g, M] view.  A block owns TW adjacent
// groups: it loads the g x TW fp16 tile with 16-byte row loads into LDS, each lane then takes
// E weights of one group from LDS; the codes go back through LDS for row-wise packed stores.
// Block = 4 waves (TW = 4 GPW groups), as on axis 1: a lane's fp64 values and the round's
// temporaries need more than 128 registers for g >= 32, and small blocks let three of them
// share a compute unit at that size.
// ------------------------------------------------------------------------------------------
template <int G>
constexpr int ax0_groups_per_block() { return 4 * Shape<G>::GPW; }
template <int G>
constexpr int ax0_threads() { return 64 * (ax0_groups_per_block<G>() / Shape<G>::GPW); }

template <int NBITS, int G, bool FIX>
__device__ __forceinline__ void ax0_tile(const SolveArgs& a, int64_t tile, int kmax, double* smem) {
  using S = Shape<G>;
  constexpr int E = S::E, L = S::L, GPW = S::GPW;
  constexpr int TW = ax0_groups_per_block<G>();  // groups per block
  constexpr int CPR = TW / 8;                    // 8-column pieces per tile row
  constexpr int ROW = TW + 8;                    // LDS row stride in halves (16-byte aligned rows)
  constexpr int NT = ax0_threads<G>();           // threads
  static_assert(NT == 256 && TW % 8 == 0 && (TW & (TW - 1)) == 0, "axis-0 block shape");
  double* meta_lds = smem;  // [2][TW]
  double* err_lds = smem + 2 * TW;  // [iters][TW]
  __half* wt = reinterpret_cast<__half*>(err_lds + (size_t)a.iters * TW);  // [G][ROW]
  uint8_t* ct = reinterpret_cast<uint8_t*>(wt);                         // [G][TW] after the loads

  const int64_t M = a.G;
  const int64_t j0 = tile * TW;
  const int tid = threadIdx.x;
  for (int task = tid; task < G * CPR; task += NT) {
    const int i = task / CPR, c = task % CPR;
    const int64_t col = j0 + 8 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < M) v = *reinterpret_cast<const uint4*>(a.W + (int64_t)i * M + col);
    *reinterpret_cast<uint4*>(wt + i * ROW + 8 * c) = v;
  }
  __syncthreads();

  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane / L, slot = lane % L;
  const int acol = wave * GPW + sub;
  const int64_t gidx = j0 + acol;
  const bool valid = gidx < M;
  double w[E], ws[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = (double)__half2float(wt[(slot * E + e) * ROW + acol]);
  __syncthreads();  // the tile is reused for the codes below

  double s, delta;
  int kfrozen;
  const double z = solve_group<E, L>(a, w, ws, valid, kmax, err_lds + acol, TW, !FIX && slot == 0, s, delta, kfrozen);
  __shared__ int s_kfrozen[4];
  if (kRecordFreeze<NBITS> && !FIX && lane == 0) s_kfrozen[wave] = kfrozen;  // published by store_block_meta

  unsigned c[E];
  final_codes<E>(ws, z, a.qmax, c);
  {
    // the same lane coordinates, formed again after the rounds (not held through them)
    const int t = late_tid();
    const int l2 = t & 63, w2 = __builtin_amdgcn_readfirstlane(t >> 6);
    const int slot2 = l2 % L, acol2 = w2 * GPW + l2 / L;
#pragma unroll
    for (int e = 0; e < E; ++e) ct[(slot2 * E + e) * TW + acol2] = (uint8_t)c[e];
    if (valid && slot2 == 0) {
      meta_lds[acol2] = delta;
      meta_lds[TW + acol2] = z;
    }
  }
  store_block_meta(a, meta_lds, TW, j0);  // its barrier also publishes the code tile
  if (kRecordFreeze<NBITS> && !FIX && threadIdx.x == 0)
    a.tile_round[tile] = max(max(s_kfrozen[0], s_kfrozen[1]), max(s_kfrozen[2], s_kfrozen[3]));
  // Rows of TW codes, 8 codes per task: flat index i*M + j0 + 8c (a multiple of 8).
  for (int task = late_tid(); task < G * CPR; task += NT) {
    const int i = task / CPR, cc = task % CPR;
    if (j0 + 8 * cc >= M) continue;
    const uint8_t* cr = ct + i * TW + 8 * cc;
    const int64_t f = (int64_t)i * M + j0 + 8 * cc;
    if constexpr (NBITS == 4) {
      unsigned word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= (unsigned)cr[e] << (4 * e);
      reinterpret_cast<unsigned*>(a.packed)[f / 8] = word;
    } else if constexpr (NBITS == 2) {
      unsigned v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (unsigned)cr[e] << (2 * e);
      reinterpret_cast<unsigned short*>(a.packed)[f / 8] = (unsigned short)v;
    } else {
      *reinterpret_cast<uint2*>(a.codes_ws + f) = *reinterpret_cast<const uint2*>(cr);
    }
  }
  if (!FIX) write_partials<TW>(a, err_lds, tile);
}

template <int NBITS, int G, bool FIX>
__global__ void __launch_bounds__(ax0_threads<G>(), solve_waves<G>()) k_quant_ax0(const SolveArgs a) {
  extern __shared__ double smem[];
  int kmax = a.iters;
  if (FIX) {
    kmax = a.ctrl[0];
    if (kmax >= a.iters) return;
  }
  for (int64_t t = blockIdx.x; t < a.nblocks; t += gridDim.x) {
    const int64_t tile = ax0_tile_of(t, a.nblocks);
    if (kRecordFreeze<NBITS> && FIX && a.tile_round[tile] <= kmax) continue;  // frozen by round kmax
    ax0_tile<NBITS, G, FIX>(a, tile, kmax, smem);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// Stop decision ("第二拍"): MAE_k = (sum of the block sums, fixed order) / N; the loop stops
// at the first k >= 1 with MAE_k not below the best so far and keeps z_(k-1) (by default;
// the rule argument picks z_(k-1), z_k or z_(k+1), and z_iters or z_(iters-1) when it never
// stops).  k_reduce and k_decide run blocks of 1024 threads.
// ------------------------------------------------------------------------------------------
// Block sums of round k are combined as a balanced pairwise tree over the blocks in index
// order, zero-padded to a power of two.  That tree splits into aligned subtrees of W = 256
// leaves: k_reduce turns each run of W entries into one entry, until at most W remain;
// k_decide forms the last tree, MAE_k = sum / N, and applies the stop rule.  Each tree is one
// wave's register butterfly (no LDS, no barrier).
constexpr int kRedThreads = 1024;
constexpr int kRedW = 256;  // entries per subtree: 64 lanes x 4

// Width of the subtrees (the same for every round count).
__host__ __device__ inline int reduce_width(int) { return kRedW; }

// Balanced pairwise tree over entries base .. base + 255 of round k of a level (zero beyond
// n_in): lane l holds entries 4l .. 4l + 3, adds them pairwise, then the DPP row steps and
// the row-pair and half-wave sums complete the tree; every lane returns the total.  Entries:
// block-major [n][iters] for the solver's per-block sums, round-major [iters][n] above.
__device__ __forceinline__ double tree256(const double* in, int64_t n_in, int64_t base, int iters, int k,
                                          bool block_major) {
  const int lane = threadIdx.x & 63;
  double v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t i = base + 4 * lane + c;
    v[c] = 0.0;
    if (i < n_in) v[c] = block_major ? in[i * iters + k] : in[(int64_t)k * n_in + i];
  }
  double x = (v[0] + v[1]) + (v[2] + v[3]);
  x = seg_sum<16>(x);
  x = add_across<true>(x);
  return add_across<false>(x);
}

// One block per run of kRedW entries; one wave per round.
__global__ void __launch_bounds__(kRedThreads) k_reduce(const double* in, int64_t n_in, double* out, int64_t n_out,
                                                        int iters, int block_major) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kRedW;
  for (int k = wave; k < iters; k += nw) {
    const double x = tree256(in, n_in, base, iters, k, block_major != 0);
    if ((threadIdx.x & 63) == 0) out[(int64_t)k * n_out + blockIdx.x] = x;
  }
}

// The last tree over the n <= kRedW entries left (zero-padded: the padding adds zeros, so the
// sums are those of the tree over next_pow2(n)), MAE_k = sum / N, and the stop rule.
__global__ void __launch_bounds__(kRedThreads) k_decide(const double* partials, int64_t n, int iters, double N,
                                                        int block_major, int stop_rule, int32_t* ctrl,
                                                        int32_t* stop_iter, double* mae_trace) {
  __shared__ double sums[HQQ_MAX_ITERS];
  __shared__ int s_rounds;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  for (int k = wave; k < iters; k += nw) {
    const double x = tree256(partials, n, 0, iters, k, block_major != 0);
    if ((threadIdx.x & 63) == 0) sums[k] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double best = __builtin_inf();
    // the rule (hqq_quantize_ex): on a stop at round k keep z_(k-1) (0), z_k (1) or z_(k+1) (2);
    // flag 4 keeps z_(iters-1) instead of z_iters when the loop never stops
    int kout = ((stop_rule & 4) && iters >= 1) ? iters - 1 : iters, rounds = iters;
    for (int k = 0; k < iters; ++k) {
      const double mae = sums[k] / N;
      if (k >= 1 && !(mae < best)) {
        kout = k - 1 + (stop_rule & 3);
        rounds = k + 1;
        break;
      }
      best = mae;
    }
    ctrl[0] = kout;
    ctrl[1] = rounds;
    if (stop_iter) *stop_iter = kout;
    s_rounds = rounds;
  }
  __syncthreads();
  if (mae_trace)
    for (int k = threadIdx.x; k < iters; k += blockDim.x) mae_trace[k] = (k < s_rounds) ? sums[k] / N : __builtin_nan("");
}

// Ten 3-bit codes per 32-bit word, bits 3t, the last word padded with code 0.
__global__ void __launch_bounds__(256) k_pack3(const uint8_t* codes, int64_t N, uint32_t* out, int64_t nwords) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nwords) return;
  uint32_t word = 0;
  const int64_t base = 10 * j;
#pragma unroll
  for (int t = 0; t < 10; ++t)
    if (base + t < N) word |= (uint32_t)codes[base + t] << (3 * t);
  out[j] = word;
}

// The words shared by neighbouring axis-1 tiles (3-bit): word T0 / 10 of tile t (T0 = t * TC not a
// multiple of 10) = the end part of tile t - 1 | the start part of tile t.
__global__ void __launch_bounds__(256) k_merge3(const uint32_t* edges, int64_t nblocks, int64_t TC, uint32_t* out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x + 1;
  if (t >= nblocks) return;
  const int64_t T0 = t * TC;
  if (T0 % 10) out[T0 / 10] = edges[2 * (t - 1) + 1] | edges[2 * t];
}

template <int NBITS, int G>
hipError_t launch_cfg(const SolveArgs& a, int axis, int64_t nblocks, int threads, size_t lds, hipStream_t st,
                      bool fix) {
  // the kernels index their tiles by a fixed block shape: refuse any other
  if (threads != (axis == 1 ? 256 : ax0_threads<G>())) return hipErrorInvalidConfiguration;
  if (axis == 1) {
    if (fix)
      hipLaunchKernelGGL((k_quant_ax1<NBITS, G, true>), dim3(nblocks), dim3(threads), lds, st, a);
    else
      hipLaunchKernelGGL((k_quant_ax1<NBITS, G, false>), dim3(nblocks), dim3(threads), lds, st, a);
  } else {
    if (fix)
      hipLaunchKernelGGL((k_quant_ax0<NBITS, G, true>), dim3(nblocks), dim3(threads), lds, st, a);
    else
      hipLaunchKernelGGL((k_quant_ax0<NBITS, G, false>), dim3(nblocks), dim3(threads), lds, st, a);
  }
  return hipGetLastError();
}

template <int NBITS>
hipError_t launch_bits(const SolveArgs& a, int g, int axis, int64_t nblocks, int threads, size_t lds,
                       hipStream_t st, bool fix) {
  switch (g) {
    case 16: return launch_cfg<NBITS, 16>(a, axis, nblocks, threads, lds, st, fix);
    case 32: return launch_cfg<NBITS, 32>(a, axis, nblocks, threads, lds, st, fix);
    case 64: return launch_cfg<NBITS, 64>(a, axis, nblocks, threads, lds, st, fix);
    case 128: return launch_cfg<NBITS, 128>(a, axis, nblocks, threads, lds, st, fix);
    case 256: return launch_cfg<NBITS, 256>(a, axis, nblocks, threads, lds, st, fix);
    default: return hipErrorInvalidValue;
  }
}

// Blocks of the fix-up grid: one 4-wave block per compute unit for each wave per SIMD the
// solve kernels are compiled for, so that a fix-up that has work runs at their occupancy.
int64_t fix_grid(int g, int64_t nblocks) {
  int waves;
  switch (g) {
    case 16: waves = solve_waves<16>(); break;
    case 32: waves = solve_waves<32>(); break;
    case 64: waves = solve_waves<64>(); break;
    case 128: waves = solve_waves<128>(); break;
    default: waves = solve_waves<256>(); break;
  }
  const int64_t full = 256 * (int64_t)waves;
  return nblocks < full ? nblocks : full;
}

int lanes_per_group(int g) {
  switch (g) {
    case 16: return Shape<16>::L;
    case 32: return Shape<32>::L;
    case 64: return Shape<64>::L;
    case 128: return Shape<128>::L;
    default: return Shape<256>::L;
  }
}

}  // namespace

bool quant_geometry(int64_t G, int g, int axis, int iters, int nbits, int64_t* nblocks, int* threads, size_t* lds) {
  if (g != 16 && g != 32 && g != 64 && g != 128 && g != 256) return false;
  const int L = lanes_per_group(g);
  const int gpw = 64 / L;
  if (axis == 1) {
    const int gpb = 4 * gpw;
    *nblocks = (G + gpb - 1) / gpb;
    *threads = 256;
    // per-round sums, steps and zeros; 3-bit: the tile's codes before packing
    *lds = (size_t)(iters + 2) * gpb * sizeof(double) + (nbits == 3 ? (size_t)gpb * g : 0);
  } else {  // the block shape of ax0_tile: tw groups, tw / gpw waves
    const int tw = 4 * gpw;
    *nblocks = (G + tw - 1) / tw;
    *threads = 64 * (tw / gpw);
    const size_t tile = (size_t)g * (tw + 8) * sizeof(__half);
    *lds = (size_t)(iters + 2) * tw * sizeof(double) + tile;
  }
  return *lds <= 64 * 1024;
}

int64_t reduce_scratch_entries(int64_t nblocks, int iters) {
  // entries of the intermediate k_reduce levels (per round)
  const int W = reduce_width(iters);
  int64_t total = 0, n = nblocks;
  while (n > W) {
    n = (n + W - 1) / W;
    total += n;
  }
  return total;
}

hipError_t launch_quantize(const SolveArgs& a, int nbits, int g, int axis, int threads, size_t lds, int64_t N,
                           int stop_rule, double* mae_trace, int32_t* stop_iter, double* reduce_ws,
                           hipStream_t st) {
  const int64_t nblocks = a.nblocks;
  hipError_t err = hipSuccess;
  auto solve = [&](bool fix, int64_t grid) {
    if (nbits == 4) return launch_bits<4>(a, g, axis, grid, threads, lds, st, fix);
    if (nbits == 3) return launch_bits<3>(a, g, axis, grid, threads, lds, st, fix);
    return launch_bits<2>(a, g, axis, grid, threads, lds, st, fix);
  };
  err = solve(false, nblocks);
  if (err != hipSuccess) return err;
  const double* level = a.partials;
  int64_t n = nblocks;
  double* next = reduce_ws;
  const int W = reduce_width(a.iters);
  int block_major = 1;  // the solver's per-block sums; later levels are round-major
  while (n > W) {
    const int64_t n_out = (n + W - 1) / W;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)n_out), dim3(kRedThreads), 0, st, level, n, next, n_out, a.iters,
                       block_major);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    level = next;
    next += n_out * a.iters;
    n = n_out;
    block_major = 0;
  }
  hipLaunchKernelGGL(k_decide, dim3(1), dim3(kRedThreads), 0, st, level, n, a.iters, (double)N, block_major,
                     stop_rule, a.ctrl, stop_iter, mae_trace);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // fix-up pass: a grid of a few blocks per compute unit (tiles in a loop), which returns at once
  // when the loop ran to the end
  err = solve(true, fix_grid(g, nblocks));
  if (err != hipSuccess) return err;
  if (nbits == 3 && axis == 1) {
    const int64_t TC = (int64_t)g * (4 * (64 / lanes_per_group(g)));  // codes per tile: g x groups per block
    if (a.nblocks > 1)
      hipLaunchKernelGGL(k_merge3, dim3((unsigned)((a.nblocks - 1 + 255) / 256)), dim3(256), 0, st, a.edges3,
                         a.nblocks, TC, reinterpret_cast<uint32_t*>(a.packed));
    err = hipGetLastError();
  } else if (nbits == 3) {
    const int64_t nwords = (N + 9) / 10;
    hipLaunchKernelGGL(k_pack3, dim3((nwords + 255) / 256), dim3(256), 0, st, a.codes_ws, N,
                       reinterpret_cast<uint32_t*>(a.packed), nwords);
    err = hipGetLastError();
  }
  return err;
}

namespace {
template <int NBITS, int G>
hipError_t launch_v2_g(const SolveArgs& a, const ScaleGrid& sg, int axis, hipStream_t st) {
  constexpr int GPB = 4 * Shape<G>::GPW;  // groups per block on either axis
  if (axis == 1) {
    hipLaunchKernelGGL((k_quant_v2<NBITS, G>), dim3((unsigned)a.nblocks), dim3(256), 2 * GPB * sizeof(double), st,
                       a, sg);
  } else {
    const size_t lds = 2 * GPB * sizeof(double) + (size_t)G * (GPB + 8) * sizeof(__half);
    hipLaunchKernelGGL((k_quant_v2_ax0<NBITS, G>), dim3((unsigned)a.nblocks), dim3(256), lds, st, a, sg);
  }
  return hipGetLastError();
}
template <int NBITS>
hipError_t launch_v2_b(const SolveArgs& a, const ScaleGrid& sg, int g, int axis, hipStream_t st) {
  switch (g) {
    case 16: return launch_v2_g<NBITS, 16>(a, sg, axis, st);
    case 32: return launch_v2_g<NBITS, 32>(a, sg, axis, st);
    case 64: return launch_v2_g<NBITS, 64>(a, sg, axis, st);
    case 128: return launch_v2_g<NBITS, 128>(a, sg, axis, st);
    case 256: return launch_v2_g<NBITS, 256>(a, sg, axis, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

int64_t quant_v2_blocks(int64_t G, int g) {
  const int gpb = 4 * (64 / lanes_per_group(g));
  return (G + gpb - 1) / gpb;
}

hipError_t launch_quantize_v2(const SolveArgs& a, const ScaleGrid& sg, int nbits, int g, int axis, hipStream_t st) {
  if (a.nblocks != quant_v2_blocks(a.G, g) || (axis != 0 && axis != 1)) return hipErrorInvalidConfiguration;
  if (nbits == 4) return launch_v2_b<4>(a, sg, g, axis, st);
  if (nbits == 2) return launch_v2_b<2>(a, sg, g, axis, st);
  if (nbits != 3 || !a.codes_ws) return hipErrorInvalidValue;
  hipError_t err = launch_v2_b<3>(a, sg, g, axis, st);
  if (err != hipSuccess) return err;
  const int64_t N = a.G * g, nwords = (N + 9) / 10;
  hipLaunchKernelGGL(k_pack3, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, st, a.codes_ws, N,
                     reinterpret_cast<uint32_t*>(a.packed), nwords);
  return hipGetLastError();
}

}  // namespace hqq
