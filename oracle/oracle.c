/*
 * oracle.c -- plain fp64 CPU reference for RMSNorm / LayerNorm forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the benchmark's
 * CPU-baseline leg, never by the GPU library.  See oracle.h for the definitions and
 * the page sections they come from.
 *
 * Everything here is the textbook definition written out, one row at a time, with
 * sequential sums in double.  No blocking, fusion or reordering: the rows are simply
 * distributed over OpenMP threads, and the column sums for dgamma / dbeta run over
 * rows 0..M-1 in order for each column, so results do not depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact decode of one stored element to double.  bfloat16 is the top half of a
 * binary32; binary16 has 1 sign, 5 exponent (bias 15) and 10 fraction bits, exponent 0
 * meaning subnormal (fraction * 2^-24) and 31 infinity or NaN. */
static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  if (dtype == ORACLE_F16) {
    const uint16_t h = ((const uint16_t*)p)[i];
    const int e = (h >> 10) & 0x1F;
    const int frac = h & 0x3FF;
    double v;
    if (e == 0) {
      v = ldexp((double)frac, -24);
    } else if (e == 31) {
      v = frac ? NAN : INFINITY;
    } else {
      v = ldexp((double)(frac + 1024), e - 25);
    }
    return (h & 0x8000) ? -v : v;
  }
  return (double)((const float*)p)[i];
}

static int64_t pick_row(const int64_t* rows, int64_t k) { return rows ? rows[k] : k; }

/* Round a double to the nearest value of the element type, ties to even: p significant
 * bits, smallest normal exponent emin, largest finite value (2 - 2^(1-p)) * 2^emax;
 * below 2^emin the spacing stays 2^(emin - p + 1) (subnormals); at or beyond the
 * midpoint between the largest finite value and 2^(emax+1) the result is infinite. */
static double round_to_type(double v, int dtype) {
  int p, emin, emax;
  if (dtype == ORACLE_BF16) {
    p = 8, emin = -126, emax = 127;
  } else if (dtype == ORACLE_F16) {
    p = 11, emin = -14, emax = 15;
  } else {
    p = 24, emin = -126, emax = 127;
  }
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  const double a = fabs(v);
  if (a >= ldexp(2.0 - ldexp(1.0, -p), emax)) return v > 0 ? INFINITY : -INFINITY;
  int k;
  frexp(a, &k); /* a = m * 2^k, 0.5 <= m < 1, so the leading bit is 2^(k-1) */
  int e = k - 1;
  if (e < emin) e = emin;
  const double q = ldexp(1.0, e - p + 1); /* spacing of the type around a */
  const double n = nearbyint(a / q);      /* exact quotient, rounded half to even */
  return copysign(n * q, v);
}

/* ---------------------------------------------------------------- statistics */

/* RMSNorm: mean of squares, add eps, reciprocal square root. */
static double rms_rstd_of_row(const void* x, int dtype, int64_t N, double eps, int64_t row) {
  const int64_t base = row * N;
  double sum_sq = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    double v = elem(x, dtype, base + j);
    sum_sq += v * v;
  }
  double mean_sq = sum_sq / (double)N;
  return 1.0 / sqrt(mean_sq + eps);
}

/* LayerNorm: mean, then the biased variance about that mean (two passes). */
static void ln_stats_of_row(const void* x, int dtype, int64_t N, double eps, int64_t row,
                            double* mean_out, double* rstd_out) {
  const int64_t base = row * N;
  double sum = 0.0;
  for (int64_t j = 0; j < N; ++j) sum += elem(x, dtype, base + j);
  double mu = sum / (double)N;
  double sum_dev_sq = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    double d = elem(x, dtype, base + j) - mu;
    sum_dev_sq += d * d;
  }
  double var = sum_dev_sq / (double)N;
  *mean_out = mu;
  *rstd_out = 1.0 / sqrt(var + eps);
}

/* ------------------------------------------------------------------ forward */

void oracle_rms_fwd(const void* x, const void* gamma, int dtype, int gdtype, int64_t N,
                    double eps, const int64_t* rows, int64_t nrows, double* y, double* rstd) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const int64_t row = pick_row(rows, k);
    const double r = rms_rstd_of_row(x, dtype, N, eps, row);
    if (rstd) rstd[k] = r;
    if (y) {
      for (int64_t j = 0; j < N; ++j) {
        y[k * N + j] = elem(x, dtype, row * N + j) * r * elem(gamma, gdtype, j);
      }
    }
  }
}

void oracle_ln_fwd(const void* x, const void* gamma, const void* beta, int dtype, int gdtype,
                   int64_t N, double eps, const int64_t* rows, int64_t nrows, double* y,
                   double* mean, double* rstd) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const int64_t row = pick_row(rows, k);
    double mu, r;
    ln_stats_of_row(x, dtype, N, eps, row, &mu, &r);
    if (mean) mean[k] = mu;
    if (rstd) rstd[k] = r;
    if (y) {
      for (int64_t j = 0; j < N; ++j) {
        double xhat = (elem(x, dtype, row * N + j) - mu) * r;
        y[k * N + j] = xhat * elem(gamma, gdtype, j) + elem(beta, gdtype, j);
      }
    }
  }
}

/* ----------------------------------------------------------------- backward */

/*
 * RMSNorm: y_j = xhat_j * gamma_j with xhat_j = x_j * r, r = (mean(x^2) + eps)^(-1/2).
 * d r / d x_k = -r^3 x_k / N, so d xhat_j / d x_k = r (delta_jk - xhat_j xhat_k / N).
 * With g_j = dy_j * gamma_j:
 *   dx_k = sum_j g_j d xhat_j / d x_k = r (g_k - xhat_k * c1),  c1 = (1/N) sum_j g_j xhat_j.
 */
void oracle_rms_bwd_dx(const void* dy, const void* x, const void* gamma, int dtype, int gdtype,
                       int64_t N, double eps, const int64_t* rows, int64_t nrows, double* dx) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const int64_t row = pick_row(rows, k);
    const int64_t base = row * N;
    const double r = rms_rstd_of_row(x, dtype, N, eps, row);
    double sum_g_xhat = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double g = elem(dy, dtype, base + j) * elem(gamma, gdtype, j);
      double xhat = elem(x, dtype, base + j) * r;
      sum_g_xhat += g * xhat;
    }
    const double c1 = sum_g_xhat / (double)N;
    for (int64_t j = 0; j < N; ++j) {
      double g = elem(dy, dtype, base + j) * elem(gamma, gdtype, j);
      double xhat = elem(x, dtype, base + j) * r;
      dx[k * N + j] = r * (g - xhat * c1);
    }
  }
}

/*
 * LayerNorm: xhat_j = (x_j - mu) r, r = (var + eps)^(-1/2), var biased.
 * d xhat_j / d x_k = r (delta_jk - 1/N - xhat_j xhat_k / N), so with g_j = dy_j gamma_j:
 *   dx_k = r (g_k - c2 - xhat_k c1),  c1 = (1/N) sum_j g_j xhat_j,  c2 = (1/N) sum_j g_j.
 */
void oracle_ln_bwd_dx(const void* dy, const void* x, const void* gamma, int dtype, int gdtype,
                      int64_t N, double eps, const int64_t* rows, int64_t nrows, double* dx) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const int64_t row = pick_row(rows, k);
    const int64_t base = row * N;
    double mu, r;
    ln_stats_of_row(x, dtype, N, eps, row, &mu, &r);
    double sum_g_xhat = 0.0, sum_g = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double g = elem(dy, dtype, base + j) * elem(gamma, gdtype, j);
      double xhat = (elem(x, dtype, base + j) - mu) * r;
      sum_g_xhat += g * xhat;
      sum_g += g;
    }
    const double c1 = sum_g_xhat / (double)N;
    const double c2 = sum_g / (double)N;
    for (int64_t j = 0; j < N; ++j) {
      double g = elem(dy, dtype, base + j) * elem(gamma, gdtype, j);
      double xhat = (elem(x, dtype, base + j) - mu) * r;
      dx[k * N + j] = r * (g - c2 - xhat * c1);
    }
  }
}

/*
 * dgamma_j = sum_i dy_ij xhat_ij (y depends on gamma_j only through the product
 * xhat_ij gamma_j); dbeta_j = sum_i dy_ij.  First the per-row statistics, then, for
 * each column, a sum over the rows 0..M-1 in order.  Each thread owns a contiguous
 * range of columns and walks the rows in order (row-major reads); the order of every
 * column's sum is the same whatever the thread count.
 */
static void column_sums(const void* dy, const void* x, int dtype, int64_t M, int64_t N,
                        const double* mu, const double* r, double* dgamma, double* dbeta,
                        double* dgamma_scale, double* dbeta_scale) {
#pragma omp parallel
  {
    int64_t nt = 1, t = 0;
#ifdef _OPENMP
    nt = omp_get_num_threads();
    t = omp_get_thread_num();
#endif
    const int64_t c0 = N * t / nt, c1 = N * (t + 1) / nt, w = c1 - c0;
    if (w > 0) {
      double* acc = (double*)calloc((size_t)(4 * w), sizeof(double));
      double *sg = acc, *sg2 = acc + w, *sb = acc + 2 * w, *sb2 = acc + 3 * w;
      for (int64_t i = 0; i < M; ++i) {
        const double m = mu ? mu[i] : 0.0;
        for (int64_t j = c0; j < c1; ++j) {
          double d = elem(dy, dtype, i * N + j);
          double xhat = (elem(x, dtype, i * N + j) - m) * r[i];
          double term = d * xhat;
          sg[j - c0] += term;
          sg2[j - c0] += term * term;
          sb[j - c0] += d;
          sb2[j - c0] += d * d;
        }
      }
      for (int64_t j = c0; j < c1; ++j) {
        if (dgamma) dgamma[j] = sg[j - c0];
        if (dgamma_scale) dgamma_scale[j] = sqrt(sg2[j - c0]);
        if (dbeta) dbeta[j] = sb[j - c0];
        if (dbeta_scale) dbeta_scale[j] = sqrt(sb2[j - c0]);
      }
      free(acc);
    }
  }
}

void oracle_rms_bwd_dgamma(const void* dy, const void* x, int dtype, int64_t M, int64_t N,
                           double eps, double* dgamma, double* dgamma_scale) {
  double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) r[i] = rms_rstd_of_row(x, dtype, N, eps, i);
  column_sums(dy, x, dtype, M, N, NULL, r, dgamma, NULL, dgamma_scale, NULL);
  free(r);
}

void oracle_ln_bwd_dgamma_dbeta(const void* dy, const void* x, int dtype, int64_t M, int64_t N,
                                double eps, double* dgamma, double* dbeta,
                                double* dgamma_scale, double* dbeta_scale) {
  size_t m = (size_t)(M > 0 ? M : 1);
  double* mu = (double*)malloc(sizeof(double) * m);
  double* r = (double*)malloc(sizeof(double) * m);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) ln_stats_of_row(x, dtype, N, eps, i, &mu[i], &r[i]);
  column_sums(dy, x, dtype, M, N, mu, r, dgamma, dbeta, dgamma_scale, dbeta_scale);
  free(mu);
  free(r);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* --------------------------------------------------------------- residual add */

/* s = x + res for the selected rows, rounded to the activation type: the stored sum
 * that a residual add in front of the norm produces and normalizes. */
void oracle_residual_sum(const void* x, const void* res, int dtype, int64_t N,
                         const int64_t* rows, int64_t nrows, double* s) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const int64_t row = pick_row(rows, k);
    for (int64_t j = 0; j < N; ++j) {
      s[k * N + j] = round_to_type(elem(x, dtype, row * N + j) + elem(res, dtype, row * N + j),
                                   dtype);
    }
  }
}
