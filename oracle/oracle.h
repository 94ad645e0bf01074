/*
 * oracle.h -- plain, slow, fp64 CPU reference for fused row normalization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * Definitions followed:
 *  - LayerNorm: subtract the row mean, divide by the row standard deviation, then
 *    scale by gamma and shift by beta ("SOTA normalization performance with
 *    torch.compile", theaicatchup.com, section "How Did Torch.compile Catch Quack?").
 *  - RMSNorm: divide the row by its root-mean-square, then scale by gamma; the steps
 *    are square, mean, add (eps), reciprocal square root, multiply, multiply
 *    ("Fused RMSNorm", aryanashta.me, section "What it is").
 *  - Backward outputs are dx, dgamma and (LayerNorm) dbeta (theaicatchup.com page,
 *    section "Why Is Peak Vectorization Your New Best Friend?").  The pages give no
 *    formulas; the ones used here are the exact derivatives of the forward.
 *
 * Inputs are raw element bits (ORACLE_F32: float, ORACLE_BF16: uint16 bfloat16,
 * ORACLE_F16: uint16 IEEE binary16), decoded exactly to double.  `dtype` is the type of
 * x and dy, `gdtype` that of gamma and beta (the "Fused RMSNorm" page, "How it works",
 * loads the row in fp16 or bf16; the parameters may be kept in fp32).  All arithmetic is in double.  Statistics are always
 * computed by the oracle from x; it never takes statistics from elsewhere.
 *
 * Row selection: `rows` lists the row indices to evaluate (into a matrix with row
 * stride N); when `rows` is NULL, rows 0 .. nrows-1 are evaluated.  Outputs are
 * packed: output row k belongs to input row rows[k].
 */
#ifndef ROWNORM_ORACLE_H
#define ROWNORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* y[k,:] (may be NULL), rstd[k] (may be NULL) */
void oracle_rms_fwd(const void* x, const void* gamma, int dtype, int gdtype, int64_t N,
                    double eps, const int64_t* rows, int64_t nrows, double* y, double* rstd);

/* y, mean, rstd each may be NULL */
void oracle_ln_fwd(const void* x, const void* gamma, const void* beta, int dtype, int gdtype,
                   int64_t N, double eps, const int64_t* rows, int64_t nrows, double* y,
                   double* mean, double* rstd);

void oracle_rms_bwd_dx(const void* dy, const void* x, const void* gamma, int dtype, int gdtype,
                       int64_t N, double eps, const int64_t* rows, int64_t nrows, double* dx);

void oracle_ln_bwd_dx(const void* dy, const void* x, const void* gamma, int dtype, int gdtype,
                      int64_t N, double eps, const int64_t* rows, int64_t nrows, double* dx);

/* Column sums over all M rows.  dgamma[j] = sum_i dy[i,j] * xhat[i,j]; for LayerNorm
 * also dbeta[j] = sum_i dy[i,j].  The *_scale outputs (may be NULL) hold
 * sqrt(sum_i t[i,j]^2) for the summed terms t, the natural size of a sum of
 * random-sign terms (used for tolerances). */
void oracle_rms_bwd_dgamma(const void* dy, const void* x, int dtype, int64_t M, int64_t N,
                           double eps, double* dgamma, double* dgamma_scale);

void oracle_ln_bwd_dgamma_dbeta(const void* dy, const void* x, int dtype, int64_t M, int64_t N,
                                double eps, double* dgamma, double* dbeta,
                                double* dgamma_scale, double* dbeta_scale);

/* Residual add in front of the norm: s[k,:] = x[row,:] + res[row,:], rounded to the
 * activation type `dtype` (nearest, ties to even).  The fused forward normalizes s and
 * stores it; the plainest reading of fusing the residual add that feeds a norm. */
void oracle_residual_sum(const void* x, const void* res, int dtype, int64_t N,
                         const int64_t* rows, int64_t nrows, double* s);

/* OpenMP threads the row loops use. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif
