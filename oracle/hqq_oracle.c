/*
 * HQQ oracle: plain, single-threaded fp64 reference.  TEST INFRASTRUCTURE ONLY
 * (see hqq_oracle.h for the sources, conventions and who may use it).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no fused multiply-add, no
 * reassociation), so every expression below is evaluated with one IEEE
 * rounding per written operation, in the written order.
 *
 * HQQ_ORACLE_PLANT selects a deliberately wrong variant of one step.  It is 0
 * in every build except the one test that checks that the pins catch such
 * mistakes.
 */
#include "hqq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifndef HQQ_ORACLE_PLANT
#define HQQ_ORACLE_PLANT 0
#endif
#define PLANT(n) (HQQ_ORACLE_PLANT == (n))

/* ------------------------------------------------------------------------------------------
 * Summation order.  The pages fix no order for the group mean or for the whole-tensor MAE;
 * every sum here is the balanced pairwise sum in index order (Higham, "The accuracy of
 * floating point summation", 1993), over the values zero-padded to the next power of two:
 * sum(v[lo .. lo+size)) = sum(first half) + sum(second half), a zero-padded half adds 0.
 * ---------------------------------------------------------------------------------------- */

static double pairwise(const double* v, int64_t lo, int64_t size, int64_t n) {
  if (lo >= n) return 0.0;
  if (size == 1) return v[lo];
  int64_t h = size / 2;
  return pairwise(v, lo, h, n) + pairwise(v, lo + h, h, n);
}

double hqq_oracle_sum(const double* v, int64_t n) {
  int64_t p = 1;
  while (p < n) p *= 2;
  if (PLANT(16)) {
    double s = 0.0;
    for (int64_t i = 0; i < n; i++) s = s + v[i];
    return s;
  }
  return pairwise(v, 0, p, n);
}

/* ------------------------------------------------------------------------------------------
 * IEEE binary16 <-> binary64
 * ---------------------------------------------------------------------------------------- */

double hqq_oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Round to nearest, ties to even. */
uint16_t hqq_oracle_double_to_half(double x) {
  if (isnan(x)) return 0x7e00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a >= 65520.0) return sign | 0x7c00; /* 65520 is the tie between 65504 and 2^16 */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: units of 2^-24; rint ties to even.  1024 units encode the
     * smallest normal number, so a carry into the exponent field is correct. */
    double units = rint(ldexp(a, 24));
    return sign | (uint16_t)units;
  }
  int e2;
  frexp(a, &e2);                /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;               /* a in [2^E, 2^(E+1)) */
  double sig = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (sig == 2048.0) {
    sig = 1024.0;
    E = E + 1;
  }
  if (E + 15 >= 31) return sign | 0x7c00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(sig - 1024.0);
}

/* ------------------------------------------------------------------------------------------
 * Group view ("axis" section: reshape([-1, g]) for axis=1, reshape([g, -1]) for axis=0,
 * statistics along `axis`).
 * ---------------------------------------------------------------------------------------- */

int64_t hqq_oracle_group_elem(int64_t rows, int64_t cols, int g, int axis, int64_t j, int i) {
  int64_t N = rows * cols;
  if (axis == 1) return j * g + i;
  if (PLANT(4)) return j * g + i;
  return (int64_t)i * (N / g) + j;
}

/* ------------------------------------------------------------------------------------------
 * Min-max start ("第一拍"): s0 = (2^b-1)/(max-min), z0 = -min*s0; s = 1 when the range is
 * too small, then s is limited to at most 2e4.  delta = 1/s is the stored step
 * ("量化公式").  `tiny` is the range at or below which s = 1 (the page gives no number).
 * ---------------------------------------------------------------------------------------- */

void hqq_oracle_init_group(const double* w, int g, int nbits, double tiny, double* s, double* delta,
                           double* z0) {
  double mn = w[0], mx = w[0];
  for (int i = 1; i < g; i++) {
    if (w[i] < mn) mn = w[i];
    if (w[i] > mx) mx = w[i];
  }
  double qmax = (double)((1 << nbits) - 1);
  if (PLANT(13)) qmax = (double)(1 << nbits);
  double d = mx - mn;
  double sv = (d <= tiny) ? 1.0 : qmax / d;
  if (sv > 2.0e4 && !PLANT(15)) sv = 2.0e4;
  *s = sv;
  *z0 = PLANT(1) ? mn * sv : -mn * sv;
  *delta = 1.0 / sv;
}

/* ------------------------------------------------------------------------------------------
 * Shrink of the residual ("shrink 不是删除极值": small residuals go to zero, large ones are
 * kept but shrunk; p = 0.7, beta = 10 by default).  Reading: the generalised soft threshold
 * e = sign(r) * max(|r| - |r|^(p-1)/beta, 0), e = 0 at r = 0.
 * ---------------------------------------------------------------------------------------- */

double hqq_oracle_shrink(double r, double beta, double p) {
  if (r == 0.0) return 0.0;
  double a = fabs(r);
  double expo = PLANT(2) ? p : p - 1.0;
  double v = a - pow(a, expo) / beta;
  if (v < 0.0) v = 0.0;
  return (r < 0.0) ? -v : v;
}

/* ------------------------------------------------------------------------------------------
 * One proximal round of one group ("第二拍", "为什么 zero 是这个均值"):
 *   q = clip(round(W*s + z), 0, 2^b-1);  W_hat = (q - z)*delta;  r = W - W_hat;
 *   err = sum |r|;  e = shrink(r);  z_next = mean(q - (W - e)*s).
 * Reading (the pages fix no evaluation order): r = W - (q - z)*delta is formed with a single
 * rounding of the product and the difference (a fused multiply-add), and the mean as
 * (sum q - sum (W - e)*s) / g, both sums pairwise in index order; the sum of the integer
 * codes is exact in any order.
 * q_out / e_out (may be NULL) receive q and e per element.
 * ---------------------------------------------------------------------------------------- */

void hqq_oracle_round_group(const double* w, int g, int nbits, double s, double delta, double z, double beta,
                            double p, double* err_sum, double* z_next, double* q_out, double* e_out) {
  double qmax = (double)((1 << nbits) - 1);
  double absr[g], qv[g], uv[g];
  for (int i = 0; i < g; i++) {
    double t = w[i] * s;
    t = t + z;
    double q = PLANT(7) ? floor(t + 0.5) : rint(t); /* rint: ties to even */
    if (q < 0.0) q = 0.0;
    if (q > qmax && !PLANT(8)) q = qmax;
    double r = fma(-(q - z), delta, w[i]); /* W - W_hat, W_hat = (q - z)*delta */
    absr[i] = fabs(r);
    double e = hqq_oracle_shrink(r, beta, p);
    uv[i] = PLANT(3) ? w[i] * s : (w[i] - e) * s;
    qv[i] = q;
    if (q_out) q_out[i] = q;
    if (e_out) e_out[i] = e;
  }
  *err_sum = hqq_oracle_sum(absr, g);
  *z_next = (hqq_oracle_sum(qv, g) - hqq_oracle_sum(uv, g)) / (double)(PLANT(12) ? g - 1 : g);
}

/* ------------------------------------------------------------------------------------------
 * Early stop ("第二拍": at most 20 rounds; when this round's reconstruction MAE is not better
 * than the best so far, go back to the previous parameters and leave the loop).
 * Readings: the best starts at +infinity; a tie is "not better"; round k's MAE is the error
 * of z_k; the parameters kept on a stop at round k* are z_(k*-1), the ones that reached the
 * best MAE; when no round stops the loop, the last update z_iters is kept.
 * ---------------------------------------------------------------------------------------- */

int hqq_oracle_stop_check(int k, double mae_k, double best) { return k >= 1 && !(mae_k < best); }

/* Index of the kept zero for a given MAE sequence (n values available) under a stop rule, and
 * the number of rounds the method evaluates.  Rules (readings of "第二拍"; 0 is the page's
 * "roll back to the previous parameters"): on a stop at round k, keep z_(k-1) (0), z_k, the
 * zero the failing round used (1), or z_(k+1), the update it computed (2); flag 4: when the
 * loop never stops, keep z_(iters-1), the last zero whose error was measured, not z_iters. */
int hqq_oracle_stop_iter_rule(const double* mae, int n, int iters, int rule, int* rounds_out) {
  double best = INFINITY;
  int limit = n < iters ? n : iters;
  for (int k = 0; k < limit; k++) {
    if (hqq_oracle_stop_check(k, mae[k], best)) {
      if (rounds_out) *rounds_out = k + 1;
      if ((rule & 3) == 0) return PLANT(6) ? k : k - 1;
      return k - 1 + (rule & 3) + (PLANT(19) && (rule & 3) == 1);
    }
    best = mae[k];
  }
  if (rounds_out) *rounds_out = limit;
  return ((rule & 4) && iters >= 1) ? iters - 1 : iters;
}

int hqq_oracle_stop_iter(const double* mae, int n, int iters, int* rounds_out) {
  return hqq_oracle_stop_iter_rule(mae, n, iters, 0, rounds_out);
}

static int valid_shape(int64_t rows, int64_t cols, int nbits, int g, int axis) {
  if (rows <= 0 || cols <= 0 || g <= 0 || nbits < 1 || nbits > 8) return 0;
  if (axis == 1) return cols % g == 0;
  if (axis == 0) return rows % g == 0;
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Whole-tensor quantisation: groups by axis, min-max start, the proximal loop with the
 * whole-tensor MAE and early stop, then one final quantisation of the original W with the
 * kept parameters ("第二拍", last sentence).
 * Outputs: codes[N] (flat row-major), s/delta/z per group (fp64), mae_out[iters] (the
 * first *rounds_out entries are set), *kout_out = index of the kept zero.
 * ---------------------------------------------------------------------------------------- */

int hqq_oracle_quantize_rule(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                             double p, double beta0, double kappa, double tiny, int stop_rule, uint8_t* codes,
                             double* s_out, double* delta_out, double* z_out, double* mae_out, int* rounds_out,
                             int* kout_out) {
  if (!valid_shape(rows, cols, nbits, g, axis) || iters < 0 || stop_rule < 0 || stop_rule > 6 ||
      (stop_rule & 3) == 3)
    return -1;
  const int64_t N = rows * cols;
  const int64_t G = N / g;
  /* The reshape of the group view, materialised group-major. */
  double* Wg = (double*)malloc((size_t)N * sizeof(double));
  double* zbuf = (double*)malloc((size_t)(3 * G) * sizeof(double));
  if (!Wg || !zbuf) {
    free(Wg);
    free(zbuf);
    return -2;
  }
  for (int64_t j = 0; j < G; j++)
    for (int i = 0; i < g; i++) Wg[j * g + i] = W[hqq_oracle_group_elem(rows, cols, g, axis, j, i)];

  double* gerr = (double*)malloc((size_t)G * sizeof(double));
  if (!gerr) {
    free(Wg);
    free(zbuf);
    return -2;
  }
  double* z_prev = zbuf;
  double* z_cur = zbuf + G;
  double* z_next = zbuf + 2 * G;
  for (int64_t j = 0; j < G; j++) hqq_oracle_init_group(Wg + j * g, g, nbits, tiny, &s_out[j], &delta_out[j], &z_cur[j]);

  double best = INFINITY;
  double beta = beta0;
  int kout = iters, rounds = 0, stopped = 0;
  const double* zk = NULL;
  for (int k = 0; k < iters; k++) {
    for (int64_t j = 0; j < G; j++)
      hqq_oracle_round_group(Wg + j * g, g, nbits, s_out[j], delta_out[j], z_cur[j], beta, p, &gerr[j], &z_next[j],
                             NULL, NULL);
    double mae = hqq_oracle_sum(gerr, G) / (double)N;
    mae_out[k] = mae;
    rounds = k + 1;
    if (hqq_oracle_stop_check(k, mae, best)) {
      /* here z_prev = z_(k-1), z_cur = z_k (this round's zero), z_next = z_(k+1) (its update) */
      const int shift = (stop_rule & 3) == 0 ? (PLANT(6) ? 1 : 0) : (stop_rule & 3) + (PLANT(19) && (stop_rule & 3) == 1);
      kout = k - 1 + shift;
      zk = shift == 0 ? z_prev : (shift == 1 ? z_cur : z_next);
      stopped = 1;
      break;
    }
    best = mae;
    double* t = z_prev;
    z_prev = z_cur;
    z_cur = z_next;
    z_next = t;
    if (!PLANT(11)) beta = beta * kappa;
  }
  /* Ran to the end: z_cur = z_iters, z_prev = z_(iters-1). */
  if (!stopped) {
    if ((stop_rule & 4) && iters >= 1) {
      kout = iters - 1;
      zk = z_prev;
    } else {
      zk = z_cur;
    }
  }

  const double qmax = (double)((1 << nbits) - 1);
  for (int64_t j = 0; j < G; j++) {
    z_out[j] = zk[j];
    for (int i = 0; i < g; i++) {
      double t = Wg[j * g + i] * s_out[j];
      t = t + zk[j];
      double q = rint(t);
      if (q < 0.0) q = 0.0;
      if (q > qmax) q = qmax;
      codes[hqq_oracle_group_elem(rows, cols, g, axis, j, i)] = (uint8_t)q;
    }
  }
  if (rounds_out) *rounds_out = rounds;
  if (kout_out) *kout_out = kout;
  free(Wg);
  free(zbuf);
  free(gerr);
  return 0;
}

int hqq_oracle_quantize(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                        double p, double beta0, double kappa, double tiny, uint8_t* codes, double* s_out,
                        double* delta_out, double* z_out, double* mae_out, int* rounds_out, int* kout_out) {
  return hqq_oracle_quantize_rule(W, rows, cols, nbits, g, axis, iters, p, beta0, kappa, tiny, 0, codes, s_out,
                                  delta_out, z_out, mae_out, rounds_out, kout_out);
}

/* ------------------------------------------------------------------------------------------
 * The same per-group steps for a list of groups with a given number of rounds `kout` (no
 * stop decision): start, kout proximal updates, final quantisation with z_kout.  Wg holds n
 * groups of g values each, in in-group order.  z_traj (n x (kout+1)) and err_traj (n x kout)
 * may be NULL.  Codes are written group-major (n x g).
 * ---------------------------------------------------------------------------------------- */

int hqq_oracle_quantize_groups(const double* Wg, int64_t n, int g, int nbits, int kout, double p, double beta0,
                               double kappa, double tiny, uint8_t* codes, double* s_out, double* delta_out,
                               double* z_out, double* z_traj, double* err_traj) {
  if (n < 0 || g <= 0 || nbits < 1 || nbits > 8 || kout < 0) return -1;
  const double qmax = (double)((1 << nbits) - 1);
  for (int64_t j = 0; j < n; j++) {
    const double* w = Wg + j * g;
    double s, delta, z;
    hqq_oracle_init_group(w, g, nbits, tiny, &s, &delta, &z);
    if (z_traj) z_traj[j * (kout + 1)] = z;
    double beta = beta0;
    for (int k = 0; k < kout; k++) {
      double err, zn;
      hqq_oracle_round_group(w, g, nbits, s, delta, z, beta, p, &err, &zn, NULL, NULL);
      if (err_traj) err_traj[j * kout + k] = err;
      z = zn;
      if (z_traj) z_traj[j * (kout + 1) + k + 1] = z;
      if (!PLANT(11)) beta = beta * kappa;
    }
    s_out[j] = s;
    delta_out[j] = delta;
    z_out[j] = z;
    for (int i = 0; i < g; i++) {
      double t = w[i] * s;
      t = t + z;
      double q = rint(t);
      if (q < 0.0) q = 0.0;
      if (q > qmax) q = qmax;
      codes[j * g + i] = (uint8_t)q;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Scale search (the slower second solver the pages name next to the default one, "第二拍":
 * it can grid-search the scale, while the default keeps the min-max scale and only refines
 * the zero).  The pages give its name and purpose only; the reading here, PARITY UNPINNED as
 * to what the reference project computes:
 *   per group (axis 1), for each multiplier c_j of a caller-given grid: s = s0 * c_j with s0
 *   the min-max start (then the same 2e4 limit), delta = 1/s, z0 = -min*s; the default
 *   proximal rounds with the default rule applied to the group's own error sum (the first
 *   k >= 1 whose sum is not below the previous one stops the loop and keeps z_(k-1); no stop
 *   keeps z_iters); the candidate's error is the pairwise sum of |W - W_hat| of its final
 *   codes.  Candidate 0 is taken first and a later one replaces it only with a strictly
 *   smaller error.  Outputs as hqq_oracle_quantize, plus the chosen index per group.
 * With one group and the grid {1} this is the default solver exactly (g is a power of two,
 * so the MAE is the error sum divided exactly).
 * ---------------------------------------------------------------------------------------- */

static double candidate_error(const double* w, int g, int nbits, double s, double delta, double z) {
  const double qmax = (double)((1 << nbits) - 1);
  double absr[g];
  for (int i = 0; i < g; i++) {
    double t = w[i] * s;
    t = t + z;
    double q = rint(t);
    if (q < 0.0) q = 0.0;
    if (q > qmax) q = qmax;
    absr[i] = fabs(w[i] - (q - z) * delta);
  }
  return hqq_oracle_sum(absr, g);
}

int hqq_oracle_quantize_v2(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                           double p, double beta0, double kappa, double tiny, const double* grid, int ncand,
                           uint8_t* codes, double* s_out, double* delta_out, double* z_out, uint8_t* choice_out) {
  if (!valid_shape(rows, cols, nbits, g, axis) || iters < 0 || ncand < 1 || ncand > 255) return -1;
  const int64_t G = rows * cols / g;
  const double qmax = (double)((1 << nbits) - 1);
  double w[g];
  for (int64_t j = 0; j < G; j++) {
    for (int i = 0; i < g; i++) w[i] = W[hqq_oracle_group_elem(rows, cols, g, axis, j, i)];
    double mn = w[0], mx = w[0];
    for (int i = 1; i < g; i++) {
      if (w[i] < mn) mn = w[i];
      if (w[i] > mx) mx = w[i];
    }
    /* the min-max start before its 2e4 limit: the multiplier scales it, then the limit */
    const double d = mx - mn;
    const double sb = (d <= tiny) ? 1.0 : qmax / d;
    double best_e = 0.0, best_s = 0.0, best_delta = 0.0, best_z = 0.0;
    int best_c = 0;
    for (int c = 0; c < ncand; c++) {
      double s = sb * grid[c];
      if (s > 2.0e4) s = 2.0e4;
      const double delta = 1.0 / s;
      double z = -mn * s;
      double zprev = z, best = INFINITY, beta = beta0;
      for (int k = 0; k < iters; k++) {
        double err, zn;
        hqq_oracle_round_group(w, g, nbits, s, delta, z, beta, p, &err, &zn, NULL, NULL);
        if (k >= 1 && !(err < best)) { /* stop: keep z_(k-1) */
          z = zprev;
          break;
        }
        best = err;
        zprev = z;
        z = zn;
        beta = beta * kappa;
      }
      const double e = candidate_error(w, g, nbits, s, delta, z);
      if (c == 0 || (PLANT(20) ? e > best_e : e < best_e)) {
        best_e = e;
        best_s = s;
        best_delta = delta;
        best_z = z;
        best_c = c;
      }
    }
    s_out[j] = best_s;
    delta_out[j] = best_delta;
    z_out[j] = best_z;
    if (choice_out) choice_out[j] = (uint8_t)best_c;
    for (int i = 0; i < g; i++) {
      double t = w[i] * best_s;
      t = t + best_z;
      double q = rint(t);
      if (q < 0.0) q = 0.0;
      if (q > qmax) q = qmax;
      codes[hqq_oracle_group_elem(rows, cols, g, axis, j, i)] = (uint8_t)q;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Bit-packing ("为什么一定要分组": two 4-bit codes per uint8, four 2-bit codes per byte, ten
 * 3-bit codes per 32-bit integer).  Reading of the layout: codes in flat row-major order,
 * little-endian within the container: 4-bit byte j = c[2j] + 16*c[2j+1]; 2-bit byte j =
 * sum_t c[4j+t]*4^t; 3-bit word j = sum_t c[10j+t]*8^t (bits 30-31 zero, the last word
 * padded with code 0), words stored little-endian.
 * ---------------------------------------------------------------------------------------- */

int64_t hqq_oracle_packed_bytes(int64_t N, int nbits) {
  if (N < 0) return -1;
  if (nbits == 4) return (N + 1) / 2;
  if (nbits == 2) return (N + 3) / 4;
  if (nbits == 3) return 4 * ((N + 9) / 10);
  return -1;
}

int hqq_oracle_pack(const uint8_t* codes, int64_t N, int nbits, uint8_t* out) {
  int64_t nb = hqq_oracle_packed_bytes(N, nbits);
  if (nb < 0) return -1;
  memset(out, 0, (size_t)nb);
  if (nbits == 4) {
    for (int64_t i = 0; i < N; i++) {
      int hi = (i % 2 == 1);
      if (PLANT(5)) hi = !hi;
      out[i / 2] |= (uint8_t)(codes[i] << (hi ? 4 : 0));
    }
  } else if (nbits == 2) {
    for (int64_t i = 0; i < N; i++) out[i / 4] |= (uint8_t)(codes[i] << (2 * (i % 4)));
  } else {
    for (int64_t j = 0; j < nb / 4; j++) {
      uint32_t word = 0;
      for (int t = 0; t < 10; t++) {
        int64_t i = 10 * j + t;
        if (i < N) word |= (uint32_t)codes[i] << (PLANT(14) ? 3 * t + 1 : 3 * t);
      }
      for (int b = 0; b < 4; b++) out[4 * j + b] = (uint8_t)(word >> (8 * b));
    }
  }
  return 0;
}

int hqq_oracle_unpack(const uint8_t* packed, int64_t N, int nbits, uint8_t* codes) {
  if (hqq_oracle_packed_bytes(N, nbits) < 0) return -1;
  if (nbits == 4) {
    for (int64_t i = 0; i < N; i++) codes[i] = (uint8_t)((packed[i / 2] >> ((i % 2) ? 4 : 0)) & 15);
  } else if (nbits == 2) {
    for (int64_t i = 0; i < N; i++) codes[i] = (uint8_t)((packed[i / 4] >> (2 * (i % 4))) & 3);
  } else {
    for (int64_t i = 0; i < N; i++) {
      int64_t j = i / 10;
      uint32_t word = (uint32_t)packed[4 * j] | ((uint32_t)packed[4 * j + 1] << 8) |
                      ((uint32_t)packed[4 * j + 2] << 16) | ((uint32_t)packed[4 * j + 3] << 24);
      codes[i] = (uint8_t)((word >> (3 * (i % 10))) & 7);
    }
  }
  return 0;
}

/* Group index of flat element `idx` (the inverse of the group view). */
static int64_t group_of(int64_t idx, int64_t rows, int64_t cols, int g, int axis) {
  int64_t N = rows * cols;
  if (axis == 1) return idx / g;
  return idx % (N / g);
}

/* ------------------------------------------------------------------------------------------
 * Dequantisation ("量化公式": W_hat = (q - z) * delta, with the stored metadata; "从压缩文件
 * 到一次前向": unpack, then (q - zero) * scale).  delta and zero are the stored values, given
 * here as doubles (exact copies of fp16 or fp32 storage).  W_hat is exact in fp64 for such
 * inputs; out_f16 receives it rounded to nearest-even.  Either output may be NULL.
 * ---------------------------------------------------------------------------------------- */

int hqq_oracle_dequant(const uint8_t* packed, const double* delta, const double* zero, int64_t rows, int64_t cols,
                       int nbits, int g, int axis, double* out_f64, uint16_t* out_f16) {
  if (!valid_shape(rows, cols, nbits, g, axis)) return -1;
  const int64_t N = rows * cols;
  uint8_t* codes = (uint8_t*)malloc((size_t)N);
  if (!codes) return -2;
  if (hqq_oracle_unpack(packed, N, nbits, codes) != 0) {
    free(codes);
    return -1;
  }
  for (int64_t idx = 0; idx < N; idx++) {
    int64_t j = group_of(idx, rows, cols, g, axis);
    double v = PLANT(9) ? ((double)codes[idx] + zero[j]) * delta[j] : ((double)codes[idx] - zero[j]) * delta[j];
    if (out_f64) out_f64[idx] = v;
    if (out_f16) out_f16[idx] = hqq_oracle_double_to_half(v);
  }
  free(codes);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * y = x @ W_hat^T ("从压缩文件到一次前向"), W [N, K] 4-bit, axis=1 groups of g along K, with
 * W_hat = (q - z) * delta from the stored metadata, all in fp64, summed in k order.
 * x is [batch, K]; y is [batch, n_sel] for the selected output rows (rows_sel == NULL selects
 * all N rows, then n_sel must equal N).
 * ---------------------------------------------------------------------------------------- */

int hqq_oracle_gemv(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K, int g,
                    const double* x, int64_t batch, const int64_t* rows_sel, int64_t n_sel, double* y) {
  if (N <= 0 || K <= 0 || g <= 0 || K % g != 0 || batch < 0) return -1;
  if (!rows_sel && n_sel != N) return -1;
  double* wrow = (double*)malloc((size_t)K * sizeof(double));
  if (!wrow) return -2;
  for (int64_t c = 0; c < n_sel; c++) {
    int64_t n = rows_sel ? rows_sel[c] : c;
    if (n < 0 || n >= N) {
      free(wrow);
      return -1;
    }
    for (int64_t k = 0; k < K; k++) {
      int64_t idx = PLANT(10) ? k * N + n : n * K + k;
      int q = (packed[idx / 2] >> ((idx % 2) ? 4 : 0)) & 15;
      int64_t j = idx / g;
      wrow[k] = ((double)q - zero[j]) * delta[j];
    }
    for (int64_t b = 0; b < batch; b++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) acc = acc + x[b * K + k] * wrow[k];
      y[b * n_sel + c] = acc;
    }
  }
  free(wrow);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * The same product for every stored format ("从压缩文件到一次前向": unpack, (q - zero) * scale,
 * x @ W_hat^T): W [N, K] with nbits in {2, 3, 4}, groups of g along K (axis 1) or the strided
 * column groups of reshape([g, -1]) (axis 0, "axis 不是一个无关紧要的开关").  Code e of the flat
 * row-major order is read straight from its container (layout reading R16), its group from the
 * group view, and the sum over k runs in k order in fp64.
 * ---------------------------------------------------------------------------------------- */

static int code_at(const uint8_t* packed, int64_t e, int nbits) {
  if (nbits == 4) return (packed[e / 2] >> ((e % 2) ? 4 : 0)) & 15;
  if (nbits == 2) return (packed[e / 4] >> (2 * (e % 4))) & 3;
  int64_t w = e / 10;
  uint32_t word = (uint32_t)packed[4 * w] | ((uint32_t)packed[4 * w + 1] << 8) | ((uint32_t)packed[4 * w + 2] << 16) |
                  ((uint32_t)packed[4 * w + 3] << 24);
  return (int)((word >> (3 * (e % 10))) & 7);
}

int hqq_oracle_gemv_fmt(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K,
                        int nbits, int g, int axis, const double* x, int64_t batch, const int64_t* rows_sel,
                        int64_t n_sel, double* y) {
  if (!valid_shape(N, K, nbits, g, axis) || nbits < 2 || nbits > 4 || batch < 0) return -1;
  if (!rows_sel && n_sel != N) return -1;
  double* wrow = (double*)malloc((size_t)K * sizeof(double));
  if (!wrow) return -2;
  for (int64_t c = 0; c < n_sel; c++) {
    int64_t n = rows_sel ? rows_sel[c] : c;
    if (n < 0 || n >= N) {
      free(wrow);
      return -1;
    }
    for (int64_t k = 0; k < K; k++) {
      int64_t e = n * K + k;
      int64_t j = PLANT(17) ? e / g : group_of(e, N, K, g, axis);
      wrow[k] = ((double)code_at(packed, e, nbits) - zero[j]) * delta[j];
    }
    for (int64_t b = 0; b < batch; b++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) acc = acc + x[b * K + k] * wrow[k];
      y[b * n_sel + c] = acc;
    }
  }
  free(wrow);
  return 0;
}

/* O9: the input gradient of the forward product, dX = dY @ W_hat ("从压缩文件到一次前向": the
 * forward is x @ W_hat^T; its gradient with respect to x multiplies by W_hat untransposed):
 * dX[b, k] = sum over n in order of dY[b, n] * (q[n, k] - z_j) * delta_j, W_hat exact in fp64,
 * for the columns k in cols_sel (all K when cols_sel is NULL; dX is [batch][n_sel]). */
int hqq_oracle_gemv_t(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K,
                      int nbits, int g, int axis, const double* dy, int64_t batch, const int64_t* cols_sel,
                      int64_t n_sel, double* dx) {
  if (!valid_shape(N, K, nbits, g, axis) || nbits < 2 || nbits > 4 || batch < 0) return -1;
  if (!cols_sel && n_sel != K) return -1;
  double* wcol = (double*)malloc((size_t)N * sizeof(double));
  if (!wcol) return -2;
  for (int64_t c = 0; c < n_sel; c++) {
    int64_t k = cols_sel ? cols_sel[c] : c;
    if (k < 0 || k >= K) {
      free(wcol);
      return -1;
    }
    for (int64_t n = 0; n < N; n++) {
      int64_t e = PLANT(18) ? (k * N + n) : (n * K + k);
      int64_t j = group_of(e, N, K, g, axis);
      wcol[n] = ((double)code_at(packed, e, nbits) - zero[j]) * delta[j];
    }
    for (int64_t b = 0; b < batch; b++) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; n++) acc = acc + dy[b * N + n] * wcol[n];
      dx[b * n_sel + c] = acc;
    }
  }
  free(wcol);
  return 0;
}

/* Array form of the fp16 rounding, for convenience. */
void hqq_oracle_doubles_to_halves(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = hqq_oracle_double_to_half(x[i]);
}
