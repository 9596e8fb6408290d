/*
 * Seeded synthetic inputs for the HQQ weight quantizer workloads.
 *
 * This module only draws numbers: it holds none of the quantizer's arithmetic.
 * Both the fp64 oracle and the GPU path are fed from the same buffers it fills.
 *
 * Generator: SplitMix64's finaliser applied to a Weyl sequence (Vigna, public
 * domain), so element i of any stream can be produced on its own and the work
 * splits over threads without changing a single value.  Normal variates use
 * the Box-Muller transform (cosine branch only, one variate per pair of
 * uniforms); Laplace variates use the inverse CDF.  The logarithm and cosine
 * are computed here with plain IEEE +,-,*,/ and sqrt (series in the reduced
 * argument), so that the values do not depend on the host's libm or on which
 * SIMD variant a library picks: the same seed gives the same bits on every
 * x86-64 machine.
 *
 * Outliers: exactly `count` distinct positions are drawn with Floyd's
 * sampling algorithm (Bentley & Floyd, CACM 1987), and each gets a fair sign.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static const uint64_t GOLDEN = 0x9E3779B97F4A7C15ULL;

/* Key of stream `stream` under `seed`: streams of one seed are unrelated. */
static uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ mix64(stream * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* Uniform on the open interval (0, 1): 53 random bits plus half a step. */
static inline double u01(uint64_t x) { return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Natural log for 0 < u < 2^1023 (normal numbers only). */
static double det_log(double u) {
  uint64_t b;
  memcpy(&b, &u, 8);
  int e = (int)((b >> 52) & 0x7ff) - 1022; /* u = m * 2^e, m in [0.5, 1) */
  b = (b & 0x000FFFFFFFFFFFFFULL) | 0x3FE0000000000000ULL;
  double m;
  memcpy(&m, &b, 8);
  if (m < 0.70710678118654752440) {
    m = m * 2.0;
    e = e - 1;
  }
  /* ln m = 2 atanh(f), f = (m-1)/(m+1), |f| <= 0.1716 */
  double f = (m - 1.0) / (m + 1.0);
  double f2 = f * f;
  double s = 1.0 / 25.0;
  for (int k = 23; k >= 1; k -= 2) s = s * f2 + 1.0 / (double)k;
  return 2.0 * f * s + (double)e * 0.69314718055994530942;
}

/* Series for cos x and sin x, |x| <= pi/4. */
static double cos_series(double x) {
  double x2 = x * x, term = 1.0, sum = 1.0;
  for (int k = 1; k <= 11; k++) {
    term = -term * x2 / (double)((2 * k - 1) * (2 * k));
    sum = sum + term;
  }
  return sum;
}
static double sin_series(double x) {
  double x2 = x * x, term = x, sum = x;
  for (int k = 1; k <= 11; k++) {
    term = -term * x2 / (double)((2 * k) * (2 * k + 1));
    sum = sum + term;
  }
  return sum;
}

/* cos(2 pi v) for 0 < v < 1, with the reduction done exactly on v. */
static double det_cos2pi(double v) {
  const double TWO_PI = 6.283185307179586476925;
  double w = v - (double)(int64_t)(v + 0.5); /* in [-0.5, 0.5] */
  if (w < 0.0) w = -w;
  double sign = 1.0;
  if (w > 0.25) {
    w = 0.5 - w;
    sign = -1.0;
  }
  if (w <= 0.125) return sign * cos_series(TWO_PI * w);
  return sign * sin_series(TWO_PI * (0.25 - w));
}

/* out[i] = mean + sigma * N(0,1) for elements start .. start+n-1 of the stream. */
void synth_normal(uint64_t seed, uint64_t stream, double mean, double sigma, int64_t start, int64_t n,
                  double* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    uint64_t idx = (uint64_t)(start + i);
    double u1 = u01(draw(key, 2 * idx));
    double u2 = u01(draw(key, 2 * idx + 1));
    double r = __builtin_sqrt(-2.0 * det_log(u1));
    out[i] = mean + sigma * (r * det_cos2pi(u2));
  }
}

/* out[i] = Laplace(0, b) by the inverse CDF: -b sgn(u-1/2) ln(1 - 2|u-1/2|). */
void synth_laplace(uint64_t seed, uint64_t stream, double b, int64_t start, int64_t n, double* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    double u = u01(draw(key, (uint64_t)(start + i)));
    double c = u - 0.5;
    double a = c < 0.0 ? -c : c;
    double l = det_log(1.0 - 2.0 * a);
    double v = -b * l;
    out[i] = c < 0.0 ? -v : v;
  }
}

/* out[i] = uniform integer in [0, bound) for i < n (bound > 0). */
void synth_randint(uint64_t seed, uint64_t stream, uint64_t bound, int64_t n, int64_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; i++) {
    unsigned __int128 p = (unsigned __int128)draw(key, (uint64_t)i) * bound;
    out[i] = (int64_t)(p >> 64);
  }
}

/*
 * Floyd's algorithm: `count` distinct positions in [0, N), returned in the
 * order they were chosen, with a sign (+1/-1) each.  Returns 0, or -1 when
 * count > N or memory is short.
 */
int synth_outliers(uint64_t seed, uint64_t stream, int64_t N, int64_t count, int64_t* pos, int8_t* sign) {
  if (count < 0 || count > N) return -1;
  uint64_t* seen = (uint64_t*)calloc((size_t)((N + 63) / 64), sizeof(uint64_t));
  if (!seen && N > 0) return -1;
  const uint64_t kpos = stream_key(seed, stream);
  const uint64_t ksign = stream_key(seed, stream + 0x5151);
  int64_t c = 0;
  for (int64_t j = N - count; j < N; j++) {
    unsigned __int128 p = (unsigned __int128)draw(kpos, (uint64_t)c) * (uint64_t)(j + 1);
    int64_t t = (int64_t)(p >> 64); /* uniform in [0, j] */
    int64_t pick = (seen[t >> 6] >> (t & 63)) & 1ULL ? j : t;
    seen[pick >> 6] |= 1ULL << (pick & 63);
    pos[c] = pick;
    sign[c] = (draw(ksign, (uint64_t)c) >> 63) ? (int8_t)-1 : (int8_t)1;
    c++;
  }
  free(seen);
  return 0;
}
