// Row-mapping planner (see plan.h).
//
// Choice of mapping, after the shape classes the autotuners fought over ("SOTA
// normalization performance with torch.compile", sections "How Did Torch.compile Catch
// Quack?" and "Why Is Peak Vectorization Your New Best Friend?": too few bytes per
// lane per load, non-power-of-2 rows such as N=384, very long rows):
//   * every lane moves whole 16-byte vectors;
//   * a row is covered by LPR lanes x VPL vectors with as little padding as possible
//     (N=384 bf16 is 48 vectors = 16 lanes x 3, one DPP row of a wavefront, no padding);
//   * among exact covers, VPL closest to a per-direction target (enough bytes in flight
//     per lane without starving occupancy), then the fewest lanes (cheaper reduction);
//   * the backward keeps per-column partial sums in registers, so it only takes mappings
//     that fit its register budget; longer rows go to the SPLIT path.
#include "plan.h"

#include "launch.h"

namespace rownorm {
namespace {

struct Mapping {
  int lpr, vpl;
};

#define RN_ENTRY(L, V) {L, V},
constexpr Mapping kFwdMappings[] = {RN_FWD_MAPPINGS(RN_ENTRY)};
constexpr Mapping kBwdMappings[] = {RN_BWD_MAPPINGS(RN_ENTRY)};
#undef RN_ENTRY

constexpr int kFwdTargetVpl = 4;
constexpr int kBwdTargetVpl = 2;
constexpr int kFwdBlocksPerCu = 8;      // 256-thread workgroups resident per CU (target)
constexpr int kBwdPartialsCap = 512;    // dgamma/dbeta partial rows of the ROWS backward
constexpr int kSplitTargetBlocks = 2048;
constexpr int kSplitMaxRowBlocks = 256;
constexpr int kRowPassMaxGrid = 2048;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <size_t K>
bool compiled(const Mapping (&list)[K], int lpr, int vpl) {
  for (const Mapping& m : list)
    if (m.lpr == lpr && m.vpl == vpl) return true;
  return false;
}

template <size_t K>
bool choose_mapping(const Mapping (&list)[K], int64_t nvec, int target, int req_lpr, int req_vpl,
                    Mapping* out) {
  bool found = false;
  Mapping best{0, 0};
  int64_t best_waste = 0;
  int best_dist = 0;
  for (const Mapping& m : list) {
    if (req_lpr && m.lpr != req_lpr) continue;
    if (req_vpl && m.vpl != req_vpl) continue;
    const int64_t cover = int64_t(m.lpr) * m.vpl;
    if (cover < nvec) continue;
    // Reject mappings where whole vector slots of every lane would be empty.
    if (cover - nvec >= m.lpr) continue;
    const int64_t waste = cover - nvec;
    const int dist = m.vpl > target ? m.vpl - target : target - m.vpl;
    const bool better = !found || waste < best_waste ||
                        (waste == best_waste && dist < best_dist) ||
                        (waste == best_waste && dist == best_dist && m.lpr < best.lpr);
    if (better) {
      found = true;
      best = m;
      best_waste = waste;
      best_dist = dist;
    }
  }
  if (found) *out = best;
  return found;
}

}  // namespace

norm_status_t make_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                        bool aligned16, const norm_options_t* opt, Plan* out) {
  norm_options_t defaults = {};
  const norm_options_t& o = opt ? *opt : defaults;
  if (o.path < NORM_PATH_AUTO || o.path > NORM_PATH_GENERIC || o.lanes_per_row < 0 ||
      o.vecs_per_lane < 0 || o.grid < 0 || o.dgamma_mode < NORM_DGAMMA_TWO_STAGE ||
      o.dgamma_mode > NORM_DGAMMA_ATOMIC_WG)
    return NORM_ERR_BAD_OPTION;
  const bool atomic = backward && o.dgamma_mode != NORM_DGAMMA_TWO_STAGE;

  Plan p;
  const int epv = dtype == NORM_DTYPE_BF16 ? 8 : 4;
  const bool vec_ok = aligned16 && (N % epv == 0);
  const int64_t nvec = vec_ok ? N / epv : 0;
  p.nvec = int(nvec);

  int path = o.path;
  Mapping m{0, 0};
  if (path == NORM_PATH_AUTO) {
    if (!vec_ok) {
      path = NORM_PATH_GENERIC;
    } else if (!backward) {
      path = choose_mapping(kFwdMappings, nvec, kFwdTargetVpl, o.lanes_per_row, o.vecs_per_lane, &m)
                 ? NORM_PATH_ROWS
                 : NORM_PATH_GENERIC;
    } else {
      path = choose_mapping(kBwdMappings, nvec, kBwdTargetVpl, o.lanes_per_row, o.vecs_per_lane, &m)
                 ? NORM_PATH_ROWS
                 : NORM_PATH_SPLIT;
    }
  } else if (path == NORM_PATH_ROWS) {
    if (!vec_ok) return NORM_ERR_BAD_OPTION;
    const bool ok = backward ? choose_mapping(kBwdMappings, nvec, kBwdTargetVpl, o.lanes_per_row,
                                              o.vecs_per_lane, &m)
                             : choose_mapping(kFwdMappings, nvec, kFwdTargetVpl, o.lanes_per_row,
                                              o.vecs_per_lane, &m);
    if (!ok) return NORM_ERR_BAD_OPTION;
  } else if (path == NORM_PATH_SPLIT) {
    if (!vec_ok || !backward) return NORM_ERR_BAD_OPTION;
  }
  if (path != NORM_PATH_ROWS && (o.lanes_per_row || o.vecs_per_lane)) return NORM_ERR_BAD_OPTION;
  if (atomic && path != NORM_PATH_ROWS) return NORM_ERR_BAD_OPTION;
  p.path = path;

  if (path == NORM_PATH_ROWS) {
    p.lpr = m.lpr;
    p.vpl = m.vpl;
    if (!backward) {
      p.block = fwd_block(m.lpr);
      p.groups = ceil_div(M, p.block / m.lpr);
      const int64_t cap = int64_t(kGfx950Cus) * (kFwdBlocksPerCu * 256 / p.block > 0
                                                     ? kFwdBlocksPerCu * 256 / p.block
                                                     : 1);
      int64_t grid = p.groups < cap ? p.groups : cap;
      if (o.grid) grid = o.grid;
      p.grid = int(grid);
    } else {
      p.block = bwd_block(m.lpr);
      p.groups = ceil_div(M, p.block / m.lpr);
      int64_t grid = p.groups < kBwdPartialsCap ? p.groups : kBwdPartialsCap;
      if (o.grid) {
        if (o.grid > grid && !atomic) return NORM_ERR_BAD_OPTION;
        grid = o.grid;
      }
      p.grid = int(grid);
      if (!atomic) {
        p.partial_rows = grid;
        p.off_part_g = 0;
        p.off_part_b = align256(size_t(grid) * size_t(N) * 4);
        p.ws_bytes = layernorm ? 2 * p.off_part_b : p.off_part_b;
      }
    }
    if (M == 0) p.grid = 0;
    *out = p;
    return NORM_OK;
  }

  if (!backward) {  // GENERIC forward
    p.block = kRowBlock;
    p.grid = int(M < kRowPassMaxGrid ? M : kRowPassMaxGrid);
    if (o.grid) p.grid = o.grid;
    if (M == 0) p.grid = 0;
    *out = p;
    return NORM_OK;
  }

  // SPLIT / GENERIC backward: row pass, column pass, column reduce.
  p.block = kSliceBlock;
  p.grid = int(M < kRowPassMaxGrid ? M : kRowPassMaxGrid);
  const int64_t slice_width = path == NORM_PATH_SPLIT ? int64_t(kSliceBlock) * kSliceVecs
                                                      : int64_t(kSliceBlock);
  const int64_t units = path == NORM_PATH_SPLIT ? nvec : N;
  p.slices = int(ceil_div(units, slice_width));
  int64_t row_blocks = ceil_div(kSplitTargetBlocks, p.slices);
  if (row_blocks > kSplitMaxRowBlocks) row_blocks = kSplitMaxRowBlocks;
  if (o.grid) row_blocks = o.grid;
  if (row_blocks > M) row_blocks = M;
  if (row_blocks < 1) row_blocks = M > 0 ? 1 : 0;
  p.rows_per_block = row_blocks ? ceil_div(M, row_blocks) : 0;
  p.partial_rows = p.rows_per_block ? ceil_div(M, p.rows_per_block) : 0;
  p.off_rowc = 0;
  p.off_part_g = align256(size_t(M) * 2 * 4);
  const size_t part = align256(size_t(p.partial_rows) * size_t(N) * 4);
  p.off_part_b = p.off_part_g + part;
  p.ws_bytes = layernorm ? p.off_part_b + part : p.off_part_b;
  if (M == 0) p.grid = 0;
  *out = p;
  return NORM_OK;
}

size_t workspace_bytes(int64_t M, int64_t N, bool layernorm, int dtype, const norm_options_t* opt) {
  size_t best = 0;
  for (int aligned = 0; aligned < 2; ++aligned) {
    Plan p;
    if (make_plan(true, layernorm, M, N, dtype, aligned != 0, opt, &p) == NORM_OK &&
        p.ws_bytes > best)
      best = p.ws_bytes;
  }
  return best;
}

}  // namespace rownorm
