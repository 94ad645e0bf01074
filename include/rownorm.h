/*
 * rownorm.h -- fused row normalization (RMSNorm and LayerNorm, forward and backward)
 * for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ types,
 * no exceptions across the boundary.
 *
 * What is computed (row i of a row-major [M, N] matrix, j = column):
 *
 *   RMSNorm forward -- "Fused RMSNorm" (aryanashta.me), section "What it is": the row
 *   is divided by its root-mean-square and scaled by gamma, the steps being square,
 *   mean, add eps, reciprocal square root, multiply, multiply:
 *       rstd_i = 1 / sqrt(mean_j(x_ij^2) + eps),   y_ij = x_ij * rstd_i * gamma_j
 *
 *   LayerNorm forward -- "SOTA normalization performance with torch.compile"
 *   (theaicatchup.com), section "How Did Torch.compile Catch Quack?": subtract the row
 *   mean, divide by the standard deviation, scale by gamma, shift by beta; the
 *   statistics are stored when the backward needs them:
 *       mean_i = mean_j(x_ij),  var_i = mean_j((x_ij - mean_i)^2) (biased),
 *       rstd_i = 1 / sqrt(var_i + eps),  y_ij = (x_ij - mean_i) * rstd_i * gamma_j + beta_j
 *
 *   Backward -- same page, section "Why Is Peak Vectorization Your New Best Friend?":
 *   the outputs are dX, dW (gamma) and, for LayerNorm, dB, with reductions over the
 *   rows of dY.  With xhat = (x - mean) * rstd (RMSNorm: x * rstd) and g = dy * gamma:
 *       c1_i = mean_j(g_ij * xhat_ij),  c2_i = mean_j(g_ij)   (LayerNorm only)
 *       dx_ij = rstd_i * (g_ij - c2_i - xhat_ij * c1_i)       (RMSNorm: no c2 term)
 *       dgamma_j = sum_i dy_ij * xhat_ij,  dbeta_j = sum_i dy_ij
 *   dgamma/dbeta are reduced in two stages without atomics (per-workgroup partial
 *   rows in a workspace, then a column-reduce kernel), the scheme "Fused RMSNorm",
 *   section "What didn't work", credits for the backward's speed.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller allocates and frees every buffer.  The library allocates
 *     no device memory and keeps no pointer after it returns.
 *   - Asynchrony: work is enqueued on `stream` (0 = the null stream); results are
 *     valid once the stream has synchronised.  The workspace must stay alive until
 *     the backward has completed on that stream.  Calls on one stream are ordered;
 *     concurrent calls on different streams must not share a workspace.
 *   - Graph capture: a call may be captured into a HIP graph (stream capture).  It
 *     enqueues kernels only (no memset, copy, allocation or synchronisation).
 *   - Errors: every argument check runs on the host before any HIP call; on an
 *     invalid argument the call returns its status and enqueues nothing.  A failed
 *     launch returns NORM_ERR_HIP.  No C++ exception crosses the boundary.
 *   - Layout: x, y, dy, dx are contiguous row-major [M, N] with row stride N; gamma
 *     and beta are [N]; mean and rstd are float [M]; dgamma and dbeta are float [N].
 *     x, y, dy, dx have the activation type of `dtype`, gamma and beta its parameter
 *     type (the same unless NORM_DTYPE_MIXED).  Element pointers must be aligned to
 *     their element size and float pointers to 4 bytes.  The fast kernels need 16-byte
 *     aligned pointers and N * sizeof(activation) a multiple of 16; other inputs run
 *     on a correct, slower scalar path.  fp16 results that exceed the fp16 range
 *     become +-inf, as a conversion of the fp32 result would.
 *   - Shapes: M >= 0, 1 <= N <= 2^31 - 1.  M = 0 is a no-op for the forward; the
 *     backward then writes zeros to dgamma/dbeta (a sum over no rows).
 *   - eps must be finite and >= 0 (eps = 0 is allowed; a constant or zero row then
 *     gives inf/NaN, as the definition does).
 *   - Outputs must not overlap inputs.  dgamma/dbeta are overwritten, not accumulated.
 *   - NaN/Inf inputs propagate: a non-finite element makes its row's outputs (and
 *     the dgamma/dbeta columns it touches) non-finite.
 */
#ifndef ROWNORM_H
#define ROWNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  The `dtype` argument of every entry point names the type of the
 * activations (x, y, dy, dx) and, by default, of gamma and beta too.  To give gamma and
 * beta a different type, pass NORM_DTYPE_MIXED(activations, parameters); supported
 * pairs: fp32/fp32, bf16/bf16, fp16/fp16, bf16 with fp32 parameters, fp16 with fp32
 * parameters (the "Fused RMSNorm" page, "How it works", loads rows in fp16 or bf16 and
 * accumulates in fp32).  Any other code or pair is NORM_ERR_BAD_DTYPE.  mean, rstd,
 * dgamma and dbeta are fp32 whatever the types. */
typedef enum norm_dtype { NORM_DTYPE_F32 = 0, NORM_DTYPE_BF16 = 1, NORM_DTYPE_F16 = 2 } norm_dtype_t;
#define NORM_DTYPE_MIXED(act, param) ((norm_dtype_t)((int)(act) | (((int)(param) + 1) << 8)))

typedef enum norm_status {
  NORM_OK = 0,
  NORM_ERR_NULL_PTR = 1,             /* a required pointer is NULL */
  NORM_ERR_BAD_SHAPE = 2,            /* M < 0, N < 1, N > 2^31-1 or M*N overflows */
  NORM_ERR_BAD_DTYPE = 3,            /* dtype is not a norm_dtype_t value */
  NORM_ERR_BAD_EPS = 4,              /* eps is negative, NaN or infinite */
  NORM_ERR_WORKSPACE_TOO_SMALL = 5,  /* workspace_bytes < the size the call needs */
  NORM_ERR_HIP = 6,                  /* a HIP runtime call or launch failed */
  NORM_ERR_MISALIGNED = 7,           /* a pointer is not aligned to its element size */
  NORM_ERR_BAD_OPTION = 8,           /* a norm_options_t field is out of range */
  NORM_ERR_SCRATCH_TOO_SMALL = 9     /* norm_ln_bwd_noalloc: the call needs more scratch
                                        than the library's static buffer holds */
} norm_status_t;

/* ------------------------------------------------------------------ forward */

/* Bytes of workspace the fastest forward plan for this shape uses, for either pointer
 * alignment: 0 except for rows long enough to be split over several workgroups, where
 * it holds their per-row partial sums (a few KiB to a few MiB), and for long rows that
 * are not whole 16-byte vectors or run past 2^17 of them (the sliced passes: 16 bytes
 * per row and slice of 2048 to 4096 elements, plus 8 per row).  The forward's workspace
 * is optional: a call given a NULL workspace or fewer bytes than its plan needs runs a
 * plan that needs none (a whole row per workgroup up to 16384 16-byte vectors, else one
 * workgroup looping over each row with element loads), slower for such rows, much
 * slower for a few very long rows, but with the same results within the stated
 * tolerances.  A pure function of its arguments: no HIP call; valid on any gfx950
 * device. */
size_t norm_fwd_workspace_size(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype);

/* RMSNorm forward.  x, gamma, y: `dtype`; rstd: float [M], or NULL to not save it.
 * workspace: NULL, or device memory, 16-byte aligned, of workspace_bytes bytes; with at
 * least norm_fwd_workspace_size(M, N, 0, dtype) bytes the fastest plan runs, else one
 * that needs no workspace (see there).  Its contents on entry do not matter and it must
 * stay alive until the call has completed on `stream`.  With the _ex variant forcing
 * NORM_PATH_CLUSTER or NORM_PATH_SPLIT the workspace is required (NORM_ERR_NULL_PTR /
 * NORM_ERR_WORKSPACE_TOO_SMALL otherwise). */
norm_status_t norm_rms_fwd(const void* x, const void* gamma, void* y, float* rstd,
                           int64_t M, int64_t N, float eps, norm_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* LayerNorm forward.  mean and rstd: float [M]; each may be NULL to not save it.
 * Workspace as above with is_layernorm = 1. */
norm_status_t norm_ln_fwd(const void* x, const void* gamma, const void* beta, void* y,
                          float* mean, float* rstd, int64_t M, int64_t N, float eps,
                          norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ----------------------------------------------------------------- backward */

/* Bytes of workspace the backward needs for this shape (0 means none).  A pure
 * function of its arguments: it makes no HIP call and is valid on any gfx950 device. */
size_t norm_bwd_workspace_size(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype);

/* RMSNorm backward.  dy, x, gamma, dx: `dtype`; rstd: the forward's saved float [M];
 * dgamma: float [N], overwritten.  workspace: device memory of at least
 * norm_bwd_workspace_size(M, N, 0, dtype) bytes, 16-byte aligned (may be NULL when
 * that size is 0).  Its contents on entry do not matter. */
norm_status_t norm_rms_bwd(const void* dy, const void* x, const void* gamma, const float* rstd,
                           void* dx, float* dgamma, int64_t M, int64_t N, norm_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* LayerNorm backward.  mean, rstd: the forward's saved float [M]; dgamma, dbeta:
 * float [N], overwritten.  Workspace as above with is_layernorm = 1. */
norm_status_t norm_ln_bwd(const void* dy, const void* x, const void* gamma, const float* mean,
                          const float* rstd, void* dx, float* dgamma, float* dbeta, int64_t M,
                          int64_t N, norm_dtype_t dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* LayerNorm backward that allocates nothing, for callers that cannot call hipMalloc
 * or take a workspace (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): norm_ln_bwd with the workspace replaced by a static device array
 * of the library's, 32 MiB per device, held from the first such call on a device until
 * the process ends.  Arguments, layouts, types, results and errors are those of
 * norm_ln_bwd.  A shape whose plan needs more scratch than that (the dgamma/dbeta
 * partial rows, 8 * N bytes per persistent workgroup, plus the split-row exchange
 * words) returns NORM_ERR_SCRATCH_TOO_SMALL before any HIP call.  Every call on one
 * device shares that device's array: calls that overlap in time on one device (on
 * different streams, or from different threads) race and give wrong dgamma/dbeta;
 * calls ordered on one stream are safe.  It makes no allocation, so it may be captured
 * into a HIP graph like the other entry points. */
norm_status_t norm_ln_bwd_noalloc(const void* dy, const void* x, const void* gamma,
                                  const float* mean, const float* rstd, void* dx, float* dgamma,
                                  float* dbeta, int64_t M, int64_t N, norm_dtype_t dtype,
                                  hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* norm_status_string(norm_status_t status);

/* ------------------------------------------------ options, plans, measurement */

/* How dgamma/dbeta are reduced over rows.  TWO_STAGE is the library's scheme.  The two
 * atomic modes exist to measure the alternative the "Fused RMSNorm" page describes in
 * its sections "How it works" and "What didn't work" (every block adding its partial
 * into one shared vector with atomics): ATOMIC_ROW adds every row's contribution
 * (M*N atomic adds), ATOMIC_WG adds one partial per workgroup (grid*N atomic adds).
 * Atomic results depend on the order of the adds and are not bitwise reproducible. */
typedef enum norm_dgamma_mode {
  NORM_DGAMMA_TWO_STAGE = 0,
  NORM_DGAMMA_ATOMIC_ROW = 1,
  NORM_DGAMMA_ATOMIC_WG = 2
} norm_dgamma_mode_t;

/* Kernel families. */
typedef enum norm_path {
  NORM_PATH_AUTO = 0,      /* the planner's choice */
  NORM_PATH_ROWS = 1,      /* register-resident rows: lanes_per_row lanes hold one row */
  NORM_PATH_SPLIT = 2,     /* the sliced passes: each row cut into column slices, every
                              pass on a (slice, row block) grid, a per-row merge between
                              them.  Forward: statistics, merge, normalize (x read
                              twice).  Backward (16-byte vectors): row sums, merge, then
                              dx and the partials (x and dy read twice).  Needs a
                              workspace in both directions */
  NORM_PATH_GENERIC = 3,   /* element loads, any N and alignment (the backward's long
                              rows take the sliced passes over elements) */
  NORM_PATH_CLUSTER = 4    /* long rows split over a cluster of workgroups, each owning
                              a column slice and exchanging per-row partial sums through
                              the workspace (a member that waits too long for another's
                              sums computes them itself, with the same result bits) */
} norm_path_t;

/* Options for the *_ex entry points; zero-initialise for defaults.  Used by tests and
 * benchmarks to force every mapping on the same inputs. */
typedef struct norm_options {
  int path;            /* norm_path_t */
  int lanes_per_row;   /* ROWS path: 8, 16, 32 or 64 (lanes of one wavefront) or 128,
                          256, 512, 1024 (one workgroup per row); 0 = planner */
  int vecs_per_lane;   /* ROWS path: 16-byte vectors each lane holds per row; 0 = planner */
  int dgamma_mode;     /* norm_dgamma_mode_t (backward only) */
  int grid;            /* persistent workgroups; 0 = planner.  For the backward this is
                          also the number of dgamma/dbeta partial rows, so size the
                          workspace with norm_bwd_workspace_size_ex and the same options.
                          CLUSTER path: total workgroups (clusters x cluster_size) */
  int cluster_size;    /* CLUSTER path: workgroups per row (2, 4, 8, 16 or 32); 0 = planner */
  int cluster_rows;    /* CLUSTER path: rows per exchange step (1 or 2); 0 = planner */
  hipEvent_t ev_start; /* if non-NULL, recorded on `stream` just before the main kernel */
  hipEvent_t ev_stop;  /* if non-NULL, recorded on `stream` just after the main kernel */
  int cluster_wait;    /* CLUSTER path: polls of another member's partial sums before
                          computing them locally; 0 = default, -1 = never wait (every
                          member computes every partial itself: for tests) */
  int pipeline;        /* ROWS path with a persistent grid (fewer workgroups than row
                          groups): 0 = planner, 1 = the plain kernel, 2 = the pipelined
                          one (two register stages, the next row group's loads in flight
                          while the current one is reduced and stored).  Ignored when every
                          workgroup takes at most one row group (the plain kernel runs);
                          the backward's pipelined kernel is two-stage mode only */
} norm_options_t;

/* What the planner chose for a call (filled by norm_plan). */
typedef struct norm_plan_info {
  int path;              /* norm_path_t actually used */
  int lanes_per_row;
  int vecs_per_lane;
  int block;             /* threads per workgroup of the main kernel */
  int grid;              /* workgroups of the main kernel */
  int partial_rows;      /* rows of dgamma/dbeta partials the backward writes */
  int cluster_size;      /* CLUSTER path: workgroups per row (else 0) */
  int cluster_rows;      /* CLUSTER path: rows per exchange step (else 0) */
  size_t workspace_bytes;
  int pipelined;         /* ROWS path: 1 if the pipelined kernel runs (see
                            norm_options_t.pipeline), else 0 */
} norm_plan_info_t;

/* Fill *info for a forward (is_backward = 0) or backward call with these arguments.
 * Pure host function; `aligned16` states whether every element pointer of the call
 * is 16-byte aligned. */
norm_status_t norm_plan(int is_backward, int is_layernorm, int64_t M, int64_t N,
                        norm_dtype_t dtype, int aligned16, const norm_options_t* opt,
                        norm_plan_info_t* info);

/* Workspace sizes for calls made with these options (NULL = defaults). */
size_t norm_fwd_workspace_size_ex(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype,
                                  const norm_options_t* opt);
size_t norm_bwd_workspace_size_ex(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype,
                                  const norm_options_t* opt);

/* Whether a call with these arguments would run on the CLUSTER path on the current
 * device: 1 yes, 0 no (another path is planned, or the device cannot hold even one
 * cluster and the call falls back to the SPLIT / GENERIC path), -1 on invalid
 * arguments.  When the device holds fewer workgroups than planned, the call runs fewer
 * clusters.  Assumes 16-byte-aligned pointers.  Makes HIP queries (current device). */
int norm_cluster_resident(int is_backward, int is_layernorm, int64_t M, int64_t N,
                          norm_dtype_t dtype, const norm_options_t* opt);

/* The entry points above with options (opt may be NULL). */
norm_status_t norm_rms_fwd_ex(const void* x, const void* gamma, void* y, float* rstd,
                              int64_t M, int64_t N, float eps, norm_dtype_t dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              const norm_options_t* opt);
norm_status_t norm_ln_fwd_ex(const void* x, const void* gamma, const void* beta, void* y,
                             float* mean, float* rstd, int64_t M, int64_t N, float eps,
                             norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, const norm_options_t* opt);
norm_status_t norm_rms_bwd_ex(const void* dy, const void* x, const void* gamma,
                              const float* rstd, void* dx, float* dgamma, int64_t M, int64_t N,
                              norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const norm_options_t* opt);
norm_status_t norm_ln_bwd_ex(const void* dy, const void* x, const void* gamma,
                             const float* mean, const float* rstd, void* dx, float* dgamma,
                             float* dbeta, int64_t M, int64_t N, norm_dtype_t dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             const norm_options_t* opt);

/* ------------------------------------------------------------ residual add fused
 * The residual add that feeds a norm, fused into it (the "SOTA normalization performance
 * with torch.compile" page credits automatic fusion of neighbouring kernels for the
 * end-to-end gains; this is the plainest such neighbour of a norm):
 *     sum = x + residual, rounded to the activation type, is written out (the updated
 *     residual stream) and is the row that is normalized: y = norm(sum).
 * In the backward, `sum` takes the place of x, and dsum (the gradient arriving at the
 * sum from its other uses; NULL means zero) is added to the result, which is then the
 * gradient of both addends:  dx = d norm(sum) / d sum (dy) + dsum.
 * Bytes: the forward also reads `residual` and writes `sum`; the backward also reads
 * `dsum`.  Everything else -- arguments, layouts, types, workspace, alignment (now
 * including residual, sum and dsum), errors -- is as for norm_*_fwd / norm_*_bwd, and
 * `opt` (may be NULL) as for the _ex variants.  sum must not overlap x or residual. */
norm_status_t norm_rms_fwd_add(const void* x, const void* residual, const void* gamma, void* y,
                               void* sum, float* rstd, int64_t M, int64_t N, float eps,
                               norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, const norm_options_t* opt);
norm_status_t norm_ln_fwd_add(const void* x, const void* residual, const void* gamma,
                              const void* beta, void* y, void* sum, float* mean, float* rstd,
                              int64_t M, int64_t N, float eps, norm_dtype_t dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              const norm_options_t* opt);
norm_status_t norm_rms_bwd_add(const void* dy, const void* sum, const void* gamma,
                               const float* rstd, const void* dsum, void* dx, float* dgamma,
                               int64_t M, int64_t N, norm_dtype_t dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream,
                               const norm_options_t* opt);
norm_status_t norm_ln_bwd_add(const void* dy, const void* sum, const void* gamma,
                              const float* mean, const float* rstd, const void* dsum, void* dx,
                              float* dgamma, float* dbeta, int64_t M, int64_t N,
                              norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const norm_options_t* opt);

/* ------------------------------------------------------------ measurement aid
 * Not part of the normalization path: the achievable-bandwidth reference the benchmark
 * quotes beside the norm kernels.  A plain streaming kernel over n 16-byte vectors with
 * the same 16-byte non-temporal loads and stores:
 *     kind 0 (copy, one read and one write per vector, the forward's mix): dst = a;
 *     kind 1 (two reads and one write, the backward's mix): dst = a + b, as 32-bit
 *     unsigned integers lane by lane.
 * a, b (kind 1 only; ignored for kind 0) and dst are device pointers aligned to 16
 * bytes; dst must not overlap a or b.  n >= 0 (n = 0 enqueues nothing).  Errors:
 * NORM_ERR_BAD_OPTION for another kind, NORM_ERR_BAD_SHAPE for n < 0,
 * NORM_ERR_NULL_PTR, NORM_ERR_MISALIGNED; a failed launch is NORM_ERR_HIP. */
norm_status_t norm_stream_reference(int kind, const void* a, const void* b, void* dst, int64_t n,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_H */
