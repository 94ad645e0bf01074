// Kernel argument blocks, the list of compiled row mappings, and the launcher
// entry points shared by the host API (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rownorm {

// ------------------------------------------------------------- element types
// Activations (x, y, dy, dx) and parameters (gamma, beta) may differ in type; these are
// the supported pairs, each built as its own set of kernels.  The public dtype code
// (rownorm.h) maps onto them in api.cpp.
enum TypeCombo {
  kTcF32 = 0,     // fp32 activations, fp32 parameters
  kTcBF16 = 1,    // bf16, bf16
  kTcF16 = 2,     // fp16, fp16
  kTcBF16F32 = 3, // bf16 activations, fp32 parameters
  kTcF16F32 = 4,  // fp16 activations, fp32 parameters
};
constexpr int kNumTypeCombos = 5;
constexpr bool tc_is16(int tc) { return tc != kTcF32; }  // 16-bit activations

// ------------------------------------------------------------ compiled mappings
// (lanes per row, 16-byte vectors per lane).  8..64 lanes: several rows per
// wavefront (a row is one aligned lane group); 128..1024 lanes: one row spans
// several wavefronts of a workgroup and is reduced through LDS.
#define RN_FWD_MAPPINGS(X)                                                             \
  X(8, 1) X(8, 2) X(8, 3) X(8, 4) X(8, 6) X(8, 8)                                      \
  X(16, 1) X(16, 2) X(16, 3) X(16, 4) X(16, 6) X(16, 8)                                \
  X(32, 1) X(32, 2) X(32, 3) X(32, 4) X(32, 6) X(32, 8)                                \
  X(64, 1) X(64, 2) X(64, 3) X(64, 4) X(64, 6) X(64, 8)                                \
  X(128, 1) X(128, 2) X(128, 3) X(128, 4) X(128, 6) X(128, 8)                          \
  X(256, 1) X(256, 2) X(256, 3) X(256, 4) X(256, 6) X(256, 8)                          \
  X(512, 1) X(512, 2) X(512, 3) X(512, 4) X(512, 6) X(512, 8)                          \
  X(1024, 1) X(1024, 2) X(1024, 3) X(1024, 4) X(1024, 5) X(1024, 6) X(1024, 7)         \
  X(1024, 8) X(512, 16) X(1024, 12) X(1024, 16)

// The backward keeps x, dy and per-column fp32 partials of dgamma (and dbeta) in
// registers.  Wide one-row workgroups keep the partials in LDS instead (bwd_lds_acc);
// 1024-lane mappings with more than one vector per lane exist only in that form (in
// registers they would exceed the 128 VGPRs a 1024-thread workgroup's lanes may use).
#define RN_BWD_MAPPINGS(X)                                                             \
  X(8, 1) X(8, 2) X(8, 3) X(8, 4)                                                      \
  X(16, 1) X(16, 2) X(16, 3) X(16, 4)                                                  \
  X(32, 1) X(32, 2) X(32, 3) X(32, 4)                                                  \
  X(64, 1) X(64, 2) X(64, 3) X(64, 4)                                                  \
  X(128, 1) X(128, 2) X(128, 3) X(128, 4)                                              \
  X(256, 1) X(256, 2) X(256, 3) X(256, 4)                                              \
  X(512, 1) X(512, 2) X(512, 3) X(512, 4)                                              \
  X(1024, 1) X(1024, 2) X(1024, 4)

constexpr int kLdsBytes = 160 * 1024;  // LDS per workgroup (and per CU) on gfx950
// fp32 partial sums per lane of a backward row mapping; epv = elements per 16-byte vector.
constexpr int bwd_acc_floats(bool ln, int epv, int vpl) { return vpl * epv * (ln ? 2 : 1); }
// Whether the backward row mapping keeps its per-column partials in LDS: one-row
// workgroups (512+ lanes) whose partials take 16 or more registers per lane, when they
// fit.  Measured on MI355X this is never slower, and it is what lets 1024-lane
// workgroups hold 2 or 4 vectors per lane (LayerNorm bf16 at N = 16384: 5.4 TB/s
// against 4.0 TB/s for the best split-row configuration).
constexpr bool bwd_lds_acc(bool ln, int epv, int lpr, int vpl) {
  return lpr >= 512 && bwd_acc_floats(ln, epv, vpl) >= 16 &&
         lpr * bwd_acc_floats(ln, epv, vpl) * 4 <= kLdsBytes;
}
// Whether the backward row mapping is built for this kind and element width.
constexpr bool bwd_mapping_built(bool ln, int epv, int lpr, int vpl) {
  return lpr < 1024 || vpl == 1 || bwd_lds_acc(ln, epv, lpr, vpl);
}

// Split-row (cluster) kernels: (threads per member workgroup, vectors per lane, rows
// per step).
#define RN_CLUSTER_FWD_MAPPINGS(X)                                                       \
  X(256, 1, 1) X(256, 2, 1) X(256, 4, 1) X(512, 1, 1) X(512, 2, 1) X(512, 4, 1)           \
  X(1024, 1, 1) X(1024, 2, 1) X(1024, 4, 1)                                              \
  X(256, 1, 2) X(256, 2, 2) X(512, 1, 2) X(512, 2, 2) X(1024, 1, 2) X(1024, 2, 2)
#define RN_CLUSTER_BWD_MAPPINGS(X)                                                       \
  X(256, 1, 1) X(256, 2, 1) X(512, 1, 1) X(512, 2, 1) X(1024, 1, 1) X(1024, 2, 1)         \
  X(256, 1, 2) X(512, 1, 2) X(1024, 1, 2) X(256, 2, 2) X(512, 2, 2)
constexpr int kMaxCluster = 32;            // workgroups sharing one row, at most
constexpr uint32_t kSpinLimit = 1u << 16;  // polls of a member's partials before a
                                           // waiting member computes them itself

// Register-resident scalar kernels (GENERIC path) for rows that are not whole 16-byte
// vectors: one row per 256-thread workgroup, this many elements per lane.  Element loads
// keep them well below the vector kernels; measured on MI355X they beat the looping
// forward (2.1-2.7 against 0.7-1.4 TB/s) up to 3072 elements and the two-pass scalar
// backward (1.6-1.9 against 1.2-1.6 TB/s) up to 1024, and lose beyond.
#define RN_GROWS_EPL(X) X(1) X(2) X(3) X(4) X(6) X(8) X(12)
constexpr int kGrowsBlock = 256;
constexpr int kGrowsFwdMaxElems = kGrowsBlock * 12;
constexpr int kGrowsBwdMaxElems = kGrowsBlock * 4;
// Smallest elements-per-lane entry of RN_GROWS_EPL covering n elements (0: none).
constexpr int grows_epl(int64_t n) {
  const int64_t e = (n + kGrowsBlock - 1) / kGrowsBlock;
  return e <= 1 ? 1 : e <= 2 ? 2 : e <= 3 ? 3 : e <= 4 ? 4 : e <= 6 ? 6 : e <= 8 ? 8
       : e <= 12 ? 12 : 0;
}

// Threads per workgroup for a row mapping.
constexpr int fwd_block(int lpr) { return lpr >= 256 ? lpr : 256; }
constexpr int bwd_block(int lpr) { return lpr >= 512 ? lpr : 512; }

// Sliced passes over rows too long for a workgroup or a cluster (split_rows.hip): a
// slice is kSliceBlock lanes x kSliceVecs 16-byte vectors, or x kSliceElems elements
// for rows that are not whole vectors.
constexpr int kSliceBlock = 256;
constexpr int kSliceVecs = 2;
constexpr int kSliceElems = 8;
constexpr int slice_units(bool vec) { return kSliceBlock * (vec ? kSliceVecs : kSliceElems); }
// Per-row merge of the slices' terms: one wavefront per row.
constexpr int kMergeBlock = 256;
// The looping scalar forward (no workspace).
constexpr int kRowBlock = 256;
// Column reduce of the partial rows: 256 threads = lanes along N x splits of the P rows.
// With many partial rows the 16-byte path gives each workgroup 8 lanes x 4 columns
// (128-byte row segments, 32 splits), so a 4096-column LayerNorm spreads over 256
// workgroups; the scalar path 32 lanes x 1 (8 splits).  Fewer partial rows than that
// take as many splits as rows.
constexpr int kColRedThreads = 256;
constexpr int colred_max_splits(bool vec4) { return vec4 ? 32 : 8; }

enum DgammaMode { kTwoStage = 0, kAtomicRow = 1, kAtomicWg = 2 };

// ------------------------------------------------------------------ arguments
struct FwdArgs {
  const void* x;
  const void* gamma;
  const void* beta;
  void* y;
  float* mean;
  float* rstd;
  int64_t M;
  int32_t N;
  int32_t nvec;    // N / elements per 16-byte vector (ROWS path)
  float eps;
  float inv_n;
  int64_t groups;  // row groups = ceil(M / rows per workgroup iteration)
  // Residual add in front of the norm (NULL when not fused): the row normalized is
  // s = x + res rounded to the activation type, and s is written to `sum`.
  const void* res;
  void* sum;
  // Pipelined kernel only: workgroups below `persistent` take row groups b, b +
  // persistent, ... below `static_end`; each workgroup above takes one of the groups
  // from static_end on (persistent = 0: every workgroup strides over all the groups).
  int64_t static_end;
  int32_t persistent;
  // SPLIT path: per-(row, slice) statistics [M, slices, 2], the merged per-row (mean,
  // rstd) [M, 2], and the (slice, row block) grid's rows per block.
  float* rowp;
  float* rowtab;
  int64_t rows_per_block;
  int32_t slices;
};

struct BwdArgs {
  const void* dy;
  const void* x;
  const void* gamma;
  const float* mean;
  const float* rstd;
  void* dx;
  float* part_g;   // [P, N] dgamma partial rows (TWO_STAGE)
  float* part_b;   // [P, N] dbeta partial rows (LayerNorm, TWO_STAGE)
  float* dgamma;   // final outputs (atomic modes add into them)
  float* dbeta;
  float* rowc;     // SPLIT / GENERIC: [M, 2] per-row (c1, c2)
  float* rowp;     // SPLIT / GENERIC: [M, slices, 2] per-(row, slice) sums of g*xhat, g
  int64_t M;
  int32_t N;
  int32_t nvec;
  float inv_n;
  int32_t mode;    // DgammaMode
  int64_t groups;
  int64_t rows_per_block;  // SPLIT / GENERIC sliced passes: rows per row block of the pass
  int32_t slices;          // SPLIT / GENERIC sliced passes: column slices
  // Gradient arriving at the residual sum from later uses (NULL when not fused): it is
  // added to dx, the gradient of both addends.
  const void* dres;
};

// Per-row merge of the sliced passes' terms (rowp [M, slices, 2]) into out [M, 2]:
// forward (mean, rstd), also stored to mean / rstd when not NULL; backward (c1, c2).
struct MergeArgs {
  const float* rowp;
  float* out;
  float* mean;
  float* rstd;
  int64_t M;
  int32_t N;
  int32_t slices;
  int32_t slice_elems;  // elements of a full slice (the last one may hold fewer)
  float inv_n;
  float eps;
};

struct ClusterArgs {
  int32_t C;                 // workgroups per row
  int32_t nclusters;         // clusters; workgroup b is member b / nclusters of cluster
                             // b % nclusters
  int32_t slice_vecs;        // 16-byte vectors of a row each member owns (nvec / C)
  int32_t rows_per_step;     // R: rows one reduction and one exchange serve
  uint32_t spin_limit;       // polls before computing a missing partial locally; 0: never poll
  unsigned long long* xchg;  // [steps][C][max(2, K)] tagged partial sums
  uint64_t tag_base;         // the call's tag base: its exchange words' tags derive from it
};

// ------------------------------------------------------------------ launchers
// kind: 0 = RMSNorm, 1 = LayerNorm.  tc: the activation/parameter type pair
// (TypeCombo).  Each returns hipErrorInvalidValue when the mapping is not compiled.
// pipe: the pipelined kernel when the grid is persistent (grid < row groups).
hipError_t launch_fwd_rows(int kind, int tc, int lpr, int vpl, const FwdArgs& a, int grid,
                           bool pipe, hipStream_t s);
hipError_t launch_bwd_rows(int kind, int tc, int lpr, int vpl, const BwdArgs& a, int grid,
                           bool pipe, hipStream_t s);
// Sliced passes (vec: 16-byte vectors, else elements) on (slices, row blocks) grids,
// with the per-row merge on merge_grid workgroups between them.  Forward: statistics,
// merge, normalize, all on row_blocks blocks of a.rows_per_block rows.  Backward: row
// sums (row_blocks blocks of rows_per_block rows), merge, then dx and the partial rows
// (col_blocks blocks of col_rows rows, one partial row each).
hipError_t launch_fwd_split(int kind, int tc, bool vec, const FwdArgs& a, int slices,
                            int row_blocks, int merge_grid, hipStream_t s);
hipError_t launch_bwd_split(int kind, int tc, bool vec, const BwdArgs& a, int slices,
                            int row_blocks, int64_t rows_per_block, int col_blocks,
                            int64_t col_rows, int merge_grid, hipStream_t s);
// Split-row kernels and their occupancy (workgroups per CU).
hipError_t launch_fwd_cluster(int kind, int tc, int t, int vpl, int rows, const FwdArgs& a,
                              const ClusterArgs& c, int grid, hipStream_t s);
hipError_t launch_bwd_cluster(int kind, int tc, int t, int vpl, int rows, const BwdArgs& a,
                              const ClusterArgs& c, int grid, hipStream_t s);
// add: the variant with the fused residual add (forward) or residual gradient (backward).
int occupancy_fwd_cluster(int kind, int tc, int t, int vpl, int rows, bool add);
int occupancy_bwd_cluster(int kind, int tc, int t, int vpl, int rows, bool add);
// GENERIC forward (scalar loads): looping kernel for any N (the plan of a call given no
// workspace), register-resident kernel (epl elements per lane, RN_GROWS_EPL) for N up
// to kGrowsFwdMaxElems; and the register-resident GENERIC backward (one partial row per
// workgroup, like the ROWS path) for N up to kGrowsBwdMaxElems.
hipError_t launch_fwd_generic(int kind, int tc, const FwdArgs& a, int grid, hipStream_t s);
hipError_t launch_fwd_grows(int kind, int tc, int epl, const FwdArgs& a, int grid, hipStream_t s);
hipError_t launch_bwd_grows(int kind, int tc, int epl, const BwdArgs& a, int grid, hipStream_t s);
// Column reduce: out[j] = sum_p part[p*N + j] for dgamma (and dbeta if part_b).
hipError_t launch_colreduce(const float* part_g, const float* part_b, int64_t P, int32_t N,
                            float* dgamma, float* dbeta, hipStream_t s);
// dgamma (and dbeta) <- 0, for the atomic modes.
hipError_t launch_zero(float* a, float* b, int32_t N, hipStream_t s);
// Measurement aid: d = a (copy) or d = a + b over n 16-byte vectors.
hipError_t launch_stream_reference(bool two_reads, const void* a, const void* b, void* d,
                                   int64_t n, hipStream_t s);

}  // namespace rownorm
