/*
 * liboracle -- plain C statement of the 4-bit codecs, for sizes where the
 * numpy oracle would take minutes.  TEST INFRASTRUCTURE ONLY: loaded by the
 * test-suite and by the CPU-baseline leg of the benchmark, never by the GPU
 * library, and it includes no header of the GPU library.
 *
 * Same definitions as the Python oracle (oracle/*.py), written again as
 * straight loops so that the two can be checked against each other:
 *
 *  - dyadic codec (DyadicGumbel page, sections 2.1, 2.2, 2.5): scale = group
 *    absmax, codes (s/8)(j-8), index = lowest j minimising |w - c_j| over the
 *    16 codes in double, all-zero group -> index 8, dequant RNE_bf16 of the
 *    exact product with a zero result stored as +0;
 *  - LUT16 codec (k-means page, sections 1.2, 2.2): levels v_j = s*L_j
 *    (exact in double), index = lowest j minimising the exact |w - v_j|;
 *  - sign + magnitude codec (int4-g32 page, sections 1.3, 2): sign = (w < 0),
 *    magnitude index = lowest j minimising the exact ||w| - M_j| (a +inf
 *    magnitude is infinitely far from every finite weight);
 *  - the 1D Lloyd fit (k-means page section 1.2; int4-g32 page section 1.3):
 *    quantile start sorted[k*stride + stride/2], then `iters` rounds of
 *    nearest-centre assignment (double, lowest index on a tie) and member
 *    mean (double sum in increasing element order); empty centres stay.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * Every function returns 0, or -1 on a shape it does not accept.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ formats */
static double bf16_val(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double f16_val(uint16_t b) {
  int s = b >> 15, e = (b >> 10) & 31, m = b & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return s ? -v : v;
}

/* Round |x| to a grid with p significant bits and subnormal quantum 2^qmin. */
static double round_grid(double a, int p, int qmin) {
  if (a == 0.0) return 0.0;
  int E;
  frexp(a, &E);          /* a = m * 2^E, m in [0.5, 1) */
  int q = E - 1 - (p - 1);
  if (q < qmin) q = qmin;
  return ldexp(nearbyint(ldexp(a, -q)), q);  /* default mode: ties to even */
}

static uint16_t rne_bf16(double x) {
  int neg = signbit(x) != 0;
  double m = round_grid(fabs(x), 8, -133);
  uint32_t u;
  if (m >= ldexp(1.0, 128)) {
    u = 0x7F800000u;
  } else {
    float f = (float)m; /* exact */
    memcpy(&u, &f, 4);
  }
  return (uint16_t)((u >> 16) | (neg ? 0x8000u : 0u));
}

static uint16_t rne_fp16(double x) {
  int neg = signbit(x) != 0;
  double m = round_grid(fabs(x), 11, -24);
  uint16_t b;
  if (m >= 65536.0) {
    b = 0x7C00;
  } else if (m < ldexp(1.0, -14)) {
    b = (uint16_t)ldexp(m, 24); /* subnormal: integer multiple of 2^-24 */
  } else {
    int E;
    double fr = frexp(m, &E);   /* m = fr * 2^E, fr in [0.5,1) */
    int e = E - 1;              /* m in [2^e, 2^(e+1)) */
    uint16_t mant = (uint16_t)(ldexp(fr, 11) - 1024.0);
    b = (uint16_t)(((e + 15) << 10) | mant);
  }
  return (uint16_t)(b | (neg ? 0x8000u : 0u));
}

/* ------------------------------------------------------------ dyadic */
int oracle_dyadic_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* idx,
                           uint16_t* scales) {
  if (k % 64) return -1;
  const int64_t g = k / 64;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t gi = 0; gi < g; ++gi) {
      const uint16_t* wg = w + r * k + gi * 64;
      double s = 0.0;
      for (int i = 0; i < 64; ++i) {
        double a = fabs(bf16_val(wg[i]));
        if (a > s) s = a;
      }
      scales[r * g + gi] = rne_bf16(s); /* s is a bf16 value: exact */
      for (int i = 0; i < 64; ++i) {
        int best = 8;
        if (s != 0.0) {
          double wi = bf16_val(wg[i]);
          double bd = INFINITY;
          for (int j = 0; j < 16; ++j) {
            double c = (s / 8.0) * (double)(j - 8);
            double d = fabs(wi - c);
            if (d < bd) { bd = d; best = j; }
          }
        }
        idx[r * k + gi * 64 + i] = (uint8_t)best;
      }
    }
  }
  return 0;
}

int oracle_dyadic_dequant(const uint8_t* idx, const uint16_t* scales, int64_t n, int64_t k,
                          uint16_t* out) {
  if (k % 64) return -1;
  const int64_t g = k / 64;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      double s = bf16_val(scales[r * g + c / 64]);
      double v = (s / 8.0) * (double)((int)idx[r * k + c] - 8);
      if (v == 0.0) v = 0.0; /* a zero result is +0 */
      out[r * k + c] = rne_bf16(v);
    }
  return 0;
}

/* ------------------------------------------------------------ nearest level */
/* Exact rounding error of a + b for finite a, b (Knuth's two-sum):
 * (a + b) - fl(a + b), itself a double.  sum = fl(a + b). */
static double two_sum_err(double a, double b, double sum) {
  const double bp = sum - a;
  const double ap = sum - bp;
  return (a - ap) + (b - bp);
}

/* Lowest index j minimising the exact |x - v[j]|, for values held exactly in
 * double (bf16 weights, products of two bf16 numbers, fp16 magnitudes, +inf).
 * The rounded distance fl(|x - v_j|) is monotone in the exact one, so only
 * the levels that share the smallest rounded distance can be the nearest.
 * Their exact distance is |h| + sgn(h) e with h = fl(x - v_j) and e the exact
 * error of that subtraction; with |h| equal for all of them, the term
 * sgn(h) e orders them exactly.  If the smallest rounded distance is +inf,
 * every level is +inf away and the lowest index wins. */
static int nearest_level(double x, const double* v, int nl) {
  int best = 0;
  double bd = fabs(x - v[0]);
  for (int j = 1; j < nl; ++j) {
    const double d = fabs(x - v[j]);
    if (d < bd) { bd = d; best = j; }
  }
  if (!isfinite(bd)) return best;
  int have = 0;
  double bk = 0.0;
  for (int j = 0; j < nl; ++j) {
    const double h = x - v[j];
    if (fabs(h) != bd) continue;
    const double e = two_sum_err(x, -v[j], h);
    const double key = h < 0.0 ? -e : e;   /* h == 0 gives e == 0 */
    if (!have || key < bk) { bk = key; best = j; have = 1; }
  }
  return best;
}

/* ------------------------------------------------------------ dyadic matmul */
/* The fp64 reference of the fused dequant-GEMV / GEMM (k-means page section
 * 4.1; DyadicGumbel page section 2.5: unpack, rebuild, multiply) for the
 * dyadic codec: y[i][r] = sum over c = 0, 1, ... of x[i][c] * w_hat[r][c],
 * every product and partial sum in double, where w_hat[r][c] is the bf16
 * value oracle_dyadic_dequant writes (RNE_bf16((s/8)(idx - 8)), a zero result
 * +0) and x is bf16 [m][k].  packed: uint8 [n][k/2] (low nibble first);
 * scales: bf16 [n][k/64]; y: double [m][n]. */
int oracle_dyadic_matmul(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                         int64_t n, int64_t k, int64_t m, double* y) {
  if (k % 64) return -1;
  const int64_t g = k / 64;
  int bad = 0;
#pragma omp parallel
  {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    if (!wrow) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      if (!wrow) continue;
      for (int64_t c = 0; c < k; ++c) {
        const int idx = (packed[r * (k / 2) + c / 2] >> (4 * (c & 1))) & 15;
        const double s = bf16_val(scales[r * g + c / 64]);
        double v = (s / 8.0) * (double)(idx - 8);
        if (v == 0.0) v = 0.0;
        wrow[c] = bf16_val(rne_bf16(v));
      }
      for (int64_t i = 0; i < m; ++i) {
        double acc = 0.0;
        for (int64_t c = 0; c < k; ++c) acc += bf16_val(x[i * k + c]) * wrow[c];
        y[i * n + r] = acc;
      }
    }
    free(wrow);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------ LUT16 */
int oracle_lut16_indices(const uint16_t* w, const uint16_t* scales, const uint16_t* lut,
                         int64_t n, int64_t k, uint8_t* idx) {
  if (k % 64) return -1;
  const int64_t g = k / 64;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t gi = 0; gi < g; ++gi) {
      double v[16];
      const double s = bf16_val(scales[r * g + gi]);
      for (int j = 0; j < 16; ++j) v[j] = s * bf16_val(lut[(r * g + gi) * 16 + j]); /* exact */
      for (int i = 0; i < 64; ++i)
        idx[r * k + gi * 64 + i] = (uint8_t)nearest_level(bf16_val(w[r * k + gi * 64 + i]), v, 16);
    }
  return 0;
}

/* ------------------------------------------------------------ sign + magnitude */
int oracle_signmag8_indices(const uint16_t* w, const uint16_t* cb, int64_t n, int64_t k,
                            uint8_t* nib) {
  if (k % 32) return -1;
  const int64_t g = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t gi = 0; gi < g; ++gi) {
      double m[8];
      for (int j = 0; j < 8; ++j) m[j] = f16_val(cb[(r * g + gi) * 8 + j]);
      for (int i = 0; i < 32; ++i) {
        const double wi = bf16_val(w[r * k + gi * 32 + i]);
        const int best = nearest_level(fabs(wi), m, 8);
        nib[r * k + gi * 32 + i] = (uint8_t)(((wi < 0.0) ? 8 : 0) | best);
      }
    }
  return 0;
}

/* ------------------------------------------------------------ 1D Lloyd */
static void sort_doubles(double* a, int n) { /* insertion sort, n <= 64 */
  for (int i = 1; i < n; ++i) {
    double v = a[i];
    int j = i - 1;
    while (j >= 0 && a[j] > v) { a[j + 1] = a[j]; --j; }
    a[j + 1] = v;
  }
}

static void lloyd1d(const double* u, int gsz, double* c, int nc, int iters) {
  double srt[64];
  memcpy(srt, u, sizeof(double) * gsz);
  sort_doubles(srt, gsz);
  const int stride = gsz / nc;
  for (int q = 0; q < nc; ++q) c[q] = srt[q * stride + stride / 2];
  int a[64];
  for (int it = 0; it < iters; ++it) {
    for (int i = 0; i < gsz; ++i) {
      int best = 0;
      double bd = fabs(u[i] - c[0]);
      for (int q = 1; q < nc; ++q) {
        double d = fabs(u[i] - c[q]);
        if (d < bd) { bd = d; best = q; }
      }
      a[i] = best;
    }
    double sum[16];
    int cnt[16];
    for (int q = 0; q < nc; ++q) { sum[q] = 0.0; cnt[q] = 0; }
    for (int i = 0; i < gsz; ++i) { sum[a[i]] += u[i]; cnt[a[i]] += 1; }
    for (int q = 0; q < nc; ++q)
      if (cnt[q] > 0) c[q] = sum[q] / (double)cnt[q];
  }
}

int oracle_lut16_fit(const uint16_t* w, int64_t n, int64_t k, int iters, uint16_t* scales,
                     uint16_t* lut) {
  if (k % 64) return -1;
  const int64_t g = k / 64;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t t = 0; t < n * g; ++t) {
    const int64_t r = t / g, gi = t % g;
    double u[64], c[16];
    double s = 0.0;
    for (int i = 0; i < 64; ++i) {
      u[i] = bf16_val(w[r * k + gi * 64 + i]);
      if (fabs(u[i]) > s) s = fabs(u[i]);
    }
    scales[t] = rne_bf16(s);
    if (s == 0.0) {
      for (int q = 0; q < 16; ++q) lut[t * 16 + q] = 0;
      continue;
    }
    for (int i = 0; i < 64; ++i) u[i] = u[i] / s;
    lloyd1d(u, 64, c, 16, iters);
    for (int q = 0; q < 16; ++q) lut[t * 16 + q] = rne_bf16(c[q]);
  }
  return 0;
}

int oracle_signmag8_fit(const uint16_t* w, int64_t n, int64_t k, int iters, uint16_t* cb) {
  if (k % 32) return -1;
  const int64_t g = k / 32;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t t = 0; t < n * g; ++t) {
    const int64_t r = t / g, gi = t % g;
    double a[32], c[8];
    for (int i = 0; i < 32; ++i) a[i] = fabs(bf16_val(w[r * k + gi * 32 + i]));
    lloyd1d(a, 32, c, 8, iters);
    for (int q = 0; q < 8; ++q) cb[t * 8 + q] = rne_fp16(c[q]);
  }
  return 0;
}

/* number of OpenMP threads a parallel region uses (reported by the benchmark),
 * and a way to change it (the benchmark times one case on a single thread) */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
