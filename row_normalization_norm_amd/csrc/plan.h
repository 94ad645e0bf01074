// Row-mapping planner: picks the kernel family, the lanes-per-row / vectors-per-lane
// mapping, the grid and the workspace layout for one call.  Pure host code (no HIP
// calls), so the same answer is available to norm_plan(), to the workspace-size queries
// and to the launch itself.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/rownorm.h"

namespace rownorm {

// Compute units of a gfx950 part (MI350X / MI355X).  Sizes persistent grids and the
// number of dgamma/dbeta partial rows; a device with fewer CUs runs the same grid with
// fewer workgroups resident at a time (the cluster path then falls back, see api.cpp).
constexpr int kGfx950Cus = 256;

struct Plan {
  int path = NORM_PATH_GENERIC;
  int lpr = 0, vpl = 0;       // ROWS: lanes per row / vectors per lane.
                              // CLUSTER: threads per member workgroup / vectors per lane.
  int block = 0;              // threads per workgroup of the main kernel
  int64_t groups = 0;         // ROWS: row groups
  int grid = 0;               // ROWS / CLUSTER: main grid; sliced passes: merge grid
  int64_t partial_rows = 0;   // P: rows of dgamma/dbeta partials (two-stage backward)
  int slices = 0;             // sliced passes: column slices (0: not a sliced plan)
  int64_t row_blocks = 0;     // sliced passes: row blocks of the forward's passes and the
  int64_t rows_per_block = 0; //   backward's first pass, and their rows per block
  int64_t col_rows_per_block = 0;  // backward column pass: rows per row block (its row
                                   // blocks are the partial rows)
  bool vec = false;           // sliced passes: 16-byte vectors (else elements)
  int nvec = 0;               // N / elements per 16-byte vector (vector paths)
  int cluster = 0;            // CLUSTER: workgroups per row
  int nclusters = 0;          // CLUSTER: clusters
  int slice_vecs = 0;         // CLUSTER: vectors per member slice
  int rows_per_step = 0;      // CLUSTER: rows one reduction and one exchange serve
  bool pipelined = false;     // ROWS: the pipelined kernel (persistent grids only)
  size_t ws_bytes = 0;        // bytes this plan uses
  size_t ws_need = 0;         // bytes the call requires (covers the fallback plan too)
  // byte offsets into the workspace: partial rows, the sliced passes' per-row table
  // (backward c1/c2, forward mean/rstd) and per-(row, slice) terms
  size_t off_part_g = 0, off_part_b = 0, off_rowc = 0, off_rowp = 0;
  size_t off_xchg = 0, xchg_bytes = 0;
};

// Returns NORM_OK or NORM_ERR_BAD_OPTION.  Shapes and dtype must already be valid; dtype
// here is the activation type (NORM_DTYPE_F32, _BF16 or _F16): the plan depends only on
// the activations' element size.
norm_status_t make_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                        bool aligned16, const norm_options_t* opt, Plan* out);

// The sliced (SPLIT) plan a CLUSTER plan falls back to when the device cannot hold one
// cluster's workgroups at once.
norm_status_t make_fallback_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                                 Plan* out);

// A forward plan that needs no workspace, for a call given none (or too little) where
// the planned one needs one (rows split over clusters, or the sliced passes): the widest
// register-resident row mapping that covers the row, else the scalar path.  The options'
// grid is kept.
norm_status_t make_fwd_plan_without_workspace(bool layernorm, int64_t M, int64_t N, int dtype,
                                              bool aligned16, const norm_options_t* opt,
                                              Plan* out);

// Workspace bytes a call needs with these options, for either pointer alignment.
size_t workspace_bytes(bool backward, int64_t M, int64_t N, bool layernorm, int dtype,
                       const norm_options_t* opt);

}  // namespace rownorm
