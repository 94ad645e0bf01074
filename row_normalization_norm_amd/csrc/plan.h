// Row-mapping planner: picks the kernel family, the lanes-per-row / vectors-per-lane
// mapping, the persistent grid and the workspace layout for one call.  Pure host code
// (no HIP calls), so the same answer is available to norm_plan(), to the workspace-size
// query and to the launch itself.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/rownorm.h"

namespace rownorm {

// Compute units of a gfx950 part (MI350X / MI355X).  Used only to size persistent grids
// and the number of dgamma/dbeta partial rows; a device with fewer CUs runs the same
// grid with fewer workgroups resident at a time.
constexpr int kGfx950Cus = 256;

struct Plan {
  int path = NORM_PATH_GENERIC;
  int lpr = 0, vpl = 0;       // ROWS mapping
  int block = 0;              // threads per workgroup of the main kernel
  int64_t groups = 0;         // ROWS: row groups
  int grid = 0;               // ROWS: persistent grid; SPLIT/GENERIC bwd: rowdot grid
  int64_t partial_rows = 0;   // P: rows of dgamma/dbeta partials (two-stage backward)
  int slices = 0;             // SPLIT/GENERIC bwd: column slices of the column pass
  int64_t rows_per_block = 0; // SPLIT/GENERIC bwd: rows per row block of the column pass
  int nvec = 0;               // N / elements per 16-byte vector (vector paths)
  size_t ws_bytes = 0;
  size_t off_part_g = 0, off_part_b = 0, off_rowc = 0;  // byte offsets into the workspace
};

// Returns NORM_OK or NORM_ERR_BAD_OPTION.  Shapes and dtype must already be valid.
norm_status_t make_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                        bool aligned16, const norm_options_t* opt, Plan* out);

// Workspace bytes a backward call needs with these options, for either pointer
// alignment (the maximum over the aligned and the scalar plan).
size_t workspace_bytes(int64_t M, int64_t N, bool layernorm, int dtype, const norm_options_t* opt);

}  // namespace rownorm
