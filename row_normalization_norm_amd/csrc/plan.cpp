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
//   * rows longer than one workgroup's register budget are split over a cluster of
//     co-resident workgroups (CLUSTER), each owning a column slice;
//   * without 16-byte alignment, or when N is not a whole number of vectors, a scalar
//     path handles any shape.
#include "plan.h"

#include "launch.h"
#include "tuned.h"

namespace rownorm {
namespace {

struct Mapping {
  int lpr, vpl;
};

#define RN_ENTRY(L, V) {L, V},
constexpr Mapping kFwdMappings[] = {RN_FWD_MAPPINGS(RN_ENTRY)};
constexpr Mapping kBwdMappings[] = {RN_BWD_MAPPINGS(RN_ENTRY)};
#undef RN_ENTRY

struct ClusterMapping {
  int t, vpl, rows;
};
#define RN_ENTRY(T, V, R) {T, V, R},
constexpr ClusterMapping kClusterFwdMappings[] = {RN_CLUSTER_FWD_MAPPINGS(RN_ENTRY)};
constexpr ClusterMapping kClusterBwdMappings[] = {RN_CLUSTER_BWD_MAPPINGS(RN_ENTRY)};
#undef RN_ENTRY

// Vectors per lane the mapping choice aims at, and the persistent grids (measured on
// MI355X across the row lengths 256..32768): the forward wants ~4 vectors (2 for rows of
// 1024+ vectors) and 512 workgroups; the backward, which also keeps per-column partial
// sums in registers, wants 2 vectors for short rows, 1 around 256 vectors and 4 beyond,
// with one workgroup per CU (two for the light 1-vector mappings).
constexpr int kFwdGrid = 512;
constexpr int kBwdGrid = 256;
int fwd_target_vpl(int64_t nvec) { return nvec < 1024 ? 4 : 2; }
int bwd_target_vpl(int64_t nvec) { return nvec <= 128 ? 2 : nvec <= 256 ? 1 : 4; }
// Longest row (in 16-byte vectors) the forward keeps in one workgroup before splitting it
// over a cluster (1024 lanes x 8 vectors), and the longest it tries the no-prefetch
// 12- and 16-vector mappings for (1024 x 16: a whole 256 KiB row per workgroup).
constexpr int64_t kFwdRowsMaxVecs = 8192;
constexpr int64_t kFwdRowsWideMaxVecs = 16384;
constexpr int64_t kBwdRowsMaxVecs = 2048;  // same for the backward
// Up to this length the backward also tries the 1024-lane mappings that keep their
// per-column partials in LDS (built for some kinds and element widths only).
constexpr int64_t kBwdRowsLdsMaxVecs = 4096;
// Vectors per lane of the cluster kernels: beyond these the kernels need more than the
// 128 VGPRs a 1024-thread workgroup may use (the backward also holds the per-column
// partial sums and a prefetched row of x and dy).
constexpr int kClusterFwdMaxVpl = 4;
constexpr int kClusterBwdMaxVpl = 2;
// Rows per cluster step: one reduction and one exchange serve this many rows.  The bf16
// backward moves half the bytes per element, so it batches two rows to amortise the
// per-step synchronisation over as many bytes as fp32 moves in one.
constexpr int kClusterFwdRows = 1;
constexpr int kClusterBwdRowsBf16 = 2;
constexpr int kClusterBwdRowsF32 = 1;
// Sliced passes.  The forward's passes and the backward's first pass aim at
// kSliceTargetBlocks workgroups with at least kSliceMinRows rows each (the per-workgroup
// set-up, gamma and beta, then serves several rows).  The backward's column pass writes
// a partial row per row block: it aims at kSplitTargetBlocks, up to kSplitMaxRowBlocks
// row blocks, or more when a block would otherwise hold over kSplitMaxBlockRows rows.
// Measured on MI355X over rows of 4 100 to 4 194 304 elements and 1 to 65 536 rows.
constexpr int kSliceTargetBlocks = 8192;
constexpr int kSliceMinRows = 4;
constexpr int kSplitTargetBlocks = 2048;
constexpr int kSplitMaxRowBlocks = 256;
constexpr int kSplitMaxBlockRows = 32;
constexpr int kMaxGridY = 65535;  // the grid's y limit
// the per-row merge's and the looping scalar forward's grid
constexpr int kRowPassMaxGrid = 2048;
// Register-resident scalar backward: workgroups (and partial rows); its element loads
// need many waves in flight.
constexpr int kGenericBwdGrid = 2048;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Best (lanes, vectors) covering `units` 16-byte vectors: least padding, then vectors per
// lane closest to `target`, then the fewest lanes (with `distance_first`, closeness to the
// target ranks before padding).  Mappings whose last vector slot would be empty in every
// lane are not considered.
template <size_t K, typename Built>
bool choose_mapping(const Mapping (&list)[K], int64_t units, int target, int max_vpl, int req_lpr,
                    int req_vpl, bool distance_first, Built built, Mapping* out) {
  bool found = false;
  Mapping best{0, 0};
  int64_t best_waste = 0;
  int best_dist = 0;
  for (const Mapping& m : list) {
    if (!built(m)) continue;
    if (req_lpr && m.lpr != req_lpr) continue;
    if (req_vpl && m.vpl != req_vpl) continue;
    if (!req_vpl && m.vpl > max_vpl) continue;
    const int64_t cover = int64_t(m.lpr) * m.vpl;
    if (cover < units || cover - units >= m.lpr) continue;
    const int64_t waste = cover - units;
    const int dist = m.vpl > target ? m.vpl - target : target - m.vpl;
    const bool fewer = m.lpr < best.lpr;
    const bool better =
        !found ||
        (distance_first
             ? (dist < best_dist || (dist == best_dist && waste < best_waste) ||
                (dist == best_dist && waste == best_waste && fewer))
             : (waste < best_waste || (waste == best_waste && dist < best_dist) ||
                (waste == best_waste && dist == best_dist && fewer)));
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

// choose_mapping over a runtime list, preferring more lanes (fewer registers per lane).
bool choose_mapping_n(const Mapping* list, int n, int64_t units, int target, int max_vpl,
                      int req_lpr, int req_vpl, Mapping* out) {
  bool found = false;
  Mapping best{0, 0};
  int64_t best_waste = 0;
  int best_dist = 0;
  for (int k = 0; k < n; ++k) {
    const Mapping& m = list[k];
    if (req_lpr && m.lpr != req_lpr) continue;
    if (req_vpl && m.vpl != req_vpl) continue;
    if (!req_vpl && m.vpl > max_vpl) continue;
    const int64_t cover = int64_t(m.lpr) * m.vpl;
    if (cover < units || cover - units >= m.lpr) continue;
    const int64_t waste = cover - units;
    const int dist = m.vpl > target ? m.vpl - target : target - m.vpl;
    const bool better = !found || waste < best_waste || (waste == best_waste && dist < best_dist) ||
                        (waste == best_waste && dist == best_dist && m.lpr > best.lpr);
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

// Whether a ROWS plan runs the pipelined kernel: only on a persistent grid (a workgroup
// takes several row groups); as the options say, else (no table entry) for rows of 128
// vectors and more, where it measured faster on MI355X than the plain kernel (shorter
// rows mostly stream better through the plain one).
constexpr int64_t kPipelineMinVecs = 128;
bool use_pipeline(const norm_options_t& o, bool persistent, int64_t nvec) {
  if (!persistent) return false;
  if (o.pipeline) return o.pipeline == 2;
  return nvec >= kPipelineMinVecs;
}

bool plan_rows(bool backward, bool layernorm, int64_t M, int64_t N, int64_t nvec,
               const norm_options_t& o, bool atomic, Plan& p) {
  Mapping m{0, 0};
  const int epv = nvec > 0 ? int(N / nvec) : 8;  // elements per 16-byte vector
  const bool ok =
      backward
          ? choose_mapping(kBwdMappings, nvec, bwd_target_vpl(nvec), 1 << 30, o.lanes_per_row,
                           o.vecs_per_lane, true,
                           [&](const Mapping& c) {
                             return bwd_mapping_built(layernorm, epv, c.lpr, c.vpl);
                           },
                           &m)
          : choose_mapping(kFwdMappings, nvec, fwd_target_vpl(nvec), 1 << 30, o.lanes_per_row,
                           o.vecs_per_lane, false, [](const Mapping&) { return true; }, &m);
  if (!ok) return false;
  p.path = NORM_PATH_ROWS;
  p.lpr = m.lpr;
  p.vpl = m.vpl;
  if (!backward) {
    p.block = fwd_block(m.lpr);
    p.groups = ceil_div(M, p.block / m.lpr);
    int64_t grid = p.groups < kFwdGrid ? p.groups : kFwdGrid;
    // An explicit grid larger than the row groups gives one group per workgroup.
    if (o.grid) grid = o.grid < p.groups ? o.grid : p.groups;
    if (grid < 1) grid = 1;
    p.grid = int(grid);
    p.pipelined = use_pipeline(o, grid < p.groups, nvec);
  } else {
    p.block = bwd_block(m.lpr);
    p.groups = ceil_div(M, p.block / m.lpr);
    const int64_t cap = (m.vpl == 1 && m.lpr >= 128) ? 2 * kBwdGrid : kBwdGrid;
    int64_t grid = p.groups < cap ? p.groups : cap;
    // An explicit grid sets the number of partial rows; the workspace size follows it
    // (norm_bwd_workspace_size_ex with the same options).
    if (o.grid) grid = o.grid < p.groups ? o.grid : p.groups;
    if (grid < 1) grid = 1;
    p.grid = int(grid);
    // the pipelined backward: two-stage mode, and registers for a second stage
    p.pipelined = !atomic && !(m.lpr == 1024 && m.vpl > 2) &&
                  use_pipeline(o, grid < p.groups, nvec);
    if (!atomic) {
      p.partial_rows = grid;
      p.off_part_g = 0;
      p.off_part_b = align256(size_t(grid) * size_t(N) * 4);
      p.ws_bytes = layernorm ? 2 * p.off_part_b : p.off_part_b;
    }
  }
  return true;
}

bool plan_cluster(bool backward, bool layernorm, int64_t M, int64_t N, int64_t nvec, int dtype,
                  const norm_options_t& o, Plan& p) {
  // the kernels index steps and rows with 32-bit integers
  if (M > int64_t(INT32_MAX) - 2) return false;
  const int max_vpl = backward ? kClusterBwdMaxVpl : kClusterFwdMaxVpl;
  const int rows = o.cluster_rows ? o.cluster_rows
                   : !backward               ? kClusterFwdRows
                   : dtype != NORM_DTYPE_F32 ? kClusterBwdRowsBf16
                                              : kClusterBwdRowsF32;
  // The compiled (threads, vectors) pairs for this rows-per-step.
  Mapping list[32];
  int n = 0;
  const ClusterMapping* all = backward ? kClusterBwdMappings : kClusterFwdMappings;
  const int count = backward ? int(sizeof(kClusterBwdMappings) / sizeof(ClusterMapping))
                             : int(sizeof(kClusterFwdMappings) / sizeof(ClusterMapping));
  for (int k = 0; k < count; ++k) {
    if (all[k].rows == rows && n < 32) list[n++] = Mapping{all[k].t, all[k].vpl};
  }
  Mapping m{0, 0};
  int C = 0;
  for (int c = 2; c <= kMaxCluster && n > 0; c *= 2) {
    if (o.cluster_size && c != o.cluster_size) continue;
    if (nvec % c) continue;
    const int64_t sv = nvec / c;
    if (choose_mapping_n(list, n, sv, max_vpl, max_vpl, o.lanes_per_row, o.vecs_per_lane, &m)) {
      C = c;
      break;
    }
  }
  if (!C) return false;
  p.rows_per_step = rows;
  p.path = NORM_PATH_CLUSTER;
  p.lpr = m.lpr;
  p.vpl = m.vpl;
  p.block = m.lpr;
  p.cluster = C;
  p.slice_vecs = int(nvec / C);
  const int per_cu = 1024 / m.lpr;  // workgroups per CU the grid assumes resident
  int64_t ncl = int64_t(kGfx950Cus) * per_cu / C;
  if (ncl >= 8) ncl -= ncl % 8;     // members of a cluster land on one XCD
  if (o.grid) ncl = o.grid / C;
  if (ncl > M) ncl = M;
  if (ncl < 1) ncl = 1;
  p.nclusters = int(ncl);
  p.grid = int(ncl * C);
  p.off_xchg = 0;
  // every step of rows has its own exchange slots: two 64-bit words per row and member
  // (a word per value, at least two per step)
  p.xchg_bytes = align256(size_t(M + rows) * C * 2 * 8);
  size_t end = p.xchg_bytes;
  if (backward) {
    p.partial_rows = ncl;
    const size_t part = align256(size_t(ncl) * size_t(N) * 4);
    p.off_part_g = end;
    p.off_part_b = end + part;
    end += layernorm ? 2 * part : part;
  }
  p.ws_bytes = end;
  return true;
}

// Row blocks of a sliced pass: the options' grid if set, else `want`, within [1, M] and
// the grid's y limit.
int64_t split_row_blocks(int64_t M, int64_t want, const norm_options_t& o) {
  int64_t rb = o.grid ? o.grid : want;
  if (rb > kMaxGridY) rb = kMaxGridY;
  if (rb > M) rb = M;
  if (rb < 1) rb = M > 0 ? 1 : 0;
  return rb;
}

// Sliced passes on a (slices, row blocks) grid for rows too long for a workgroup or a
// cluster, and for long rows that are not whole vectors: the forward (SPLIT) and the
// backward (SPLIT for 16-byte vectors, else GENERIC with vpl = 0).  Workspace: the
// per-row table [M, 2], the per-(row, slice) terms [M, slices, 2], then the backward's
// partial rows (one per row block of its column pass).
void plan_split(bool backward, bool layernorm, int64_t M, int64_t N, int64_t nvec, bool vec,
                const norm_options_t& o, Plan& p) {
  p.path = (vec || !backward) ? NORM_PATH_SPLIT : NORM_PATH_GENERIC;
  p.vec = vec;
  p.block = kSliceBlock;
  const int64_t merge_blocks = ceil_div(M, kMergeBlock / 64);
  p.grid = int(merge_blocks < kRowPassMaxGrid ? merge_blocks : kRowPassMaxGrid);
  p.slices = int(ceil_div(vec ? nvec : N, slice_units(vec)));
  int64_t want = ceil_div(kSliceTargetBlocks, p.slices);
  if (want > ceil_div(M, kSliceMinRows)) want = ceil_div(M, kSliceMinRows);
  const int64_t rb = split_row_blocks(M, want, o);
  p.rows_per_block = rb ? ceil_div(M, rb) : 0;
  p.row_blocks = p.rows_per_block ? ceil_div(M, p.rows_per_block) : 0;
  p.off_rowc = 0;
  p.off_rowp = align256(size_t(M) * 2 * 4);
  size_t end = p.off_rowp + align256(size_t(M) * size_t(p.slices) * 2 * 4);
  if (backward) {
    int64_t cwant = ceil_div(kSplitTargetBlocks, p.slices);
    int64_t cmax = ceil_div(M, kSplitMaxBlockRows);
    if (cmax < kSplitMaxRowBlocks) cmax = kSplitMaxRowBlocks;
    if (cwant > cmax) cwant = cmax;
    const int64_t cb = split_row_blocks(M, cwant, o);
    p.col_rows_per_block = cb ? ceil_div(M, cb) : 0;
    p.partial_rows = p.col_rows_per_block ? ceil_div(M, p.col_rows_per_block) : 0;
    const size_t part = align256(size_t(p.partial_rows) * size_t(N) * 4);
    p.off_part_g = end;
    p.off_part_b = end + part;
    end += layernorm ? 2 * part : part;
  }
  p.ws_bytes = end;
}

// GENERIC forward: the register-resident scalar kernel (vpl = elements per lane) for rows
// up to kGrowsFwdMaxElems, else the looping kernel (vpl = 0), which needs no workspace.
void plan_generic_fwd(int64_t M, int64_t N, const norm_options_t& o, Plan& p) {
  p.path = NORM_PATH_GENERIC;
  p.block = kRowBlock;
  p.vpl = N <= kGrowsFwdMaxElems ? grows_epl(N) : 0;
  p.lpr = p.vpl ? kGrowsBlock : 0;
  p.grid = int(M < kRowPassMaxGrid ? M : kRowPassMaxGrid);
  if (o.grid) p.grid = o.grid;
}

// GENERIC backward: the register-resident scalar kernel with one dgamma/dbeta partial row
// per workgroup for rows up to kGrowsBwdMaxElems, else the scalar split path.
void plan_generic_bwd(bool layernorm, int64_t M, int64_t N, int64_t nvec, bool atomic,
                      const norm_options_t& o, Plan& p) {
  const int epl = N <= kGrowsBwdMaxElems ? grows_epl(N) : 0;
  if (!epl) {
    plan_split(true, layernorm, M, N, nvec, false, o, p);
    return;
  }
  p.path = NORM_PATH_GENERIC;
  p.block = kGrowsBlock;
  p.lpr = kGrowsBlock;
  p.vpl = epl;
  int64_t grid = M < kGenericBwdGrid ? M : kGenericBwdGrid;
  if (o.grid) grid = o.grid < M ? o.grid : M;
  if (grid < 1) grid = 1;
  p.grid = int(grid);
  if (!atomic) {
    p.partial_rows = grid;
    p.off_part_g = 0;
    p.off_part_b = align256(size_t(grid) * size_t(N) * 4);
    p.ws_bytes = layernorm ? 2 * p.off_part_b : p.off_part_b;
  }
}

const TunedPlan* find_tuned(bool backward, bool layernorm, int dtype, int64_t nvec) {
  for (const TunedPlan& t : kTunedPlans) {
    if (t.backward == int(backward) && t.layernorm == int(layernorm) &&
        t.bf16 == int(dtype != NORM_DTYPE_F32) && t.nvec == nvec)
      return &t;
  }
  return nullptr;
}

}  // namespace

norm_status_t make_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                        bool aligned16, const norm_options_t* opt, Plan* out) {
  norm_options_t defaults = {};
  const norm_options_t& o = opt ? *opt : defaults;
  if (o.path < NORM_PATH_AUTO || o.path > NORM_PATH_CLUSTER || o.lanes_per_row < 0 ||
      o.vecs_per_lane < 0 || o.grid < 0 || o.cluster_size < 0 || o.cluster_size > kMaxCluster ||
      o.cluster_rows < 0 || o.cluster_rows > 2 ||
      o.dgamma_mode < NORM_DGAMMA_TWO_STAGE || o.dgamma_mode > NORM_DGAMMA_ATOMIC_WG ||
      o.pipeline < 0 || o.pipeline > 2)
    return NORM_ERR_BAD_OPTION;
  const bool atomic = backward && o.dgamma_mode != NORM_DGAMMA_TWO_STAGE;

  Plan p;
  const int epv = dtype != NORM_DTYPE_F32 ? 8 : 4;
  const bool vec_ok = aligned16 && (N % epv == 0);
  const int64_t nvec = vec_ok ? N / epv : 0;
  p.nvec = int(nvec);

  bool ok = true;
  switch (o.path) {
    case NORM_PATH_AUTO:
      if (const TunedPlan* t = (vec_ok && !atomic && !o.lanes_per_row && !o.vecs_per_lane &&
                                !o.cluster_size && !o.cluster_rows)
                                   ? find_tuned(backward, layernorm, dtype, nvec)
                                   : nullptr) {
        norm_options_t ot = o;
        ot.lanes_per_row = t->lanes;
        ot.vecs_per_lane = t->vecs;
        if (!ot.grid) ot.grid = t->grid;
        if (!ot.pipeline) ot.pipeline = t->pipelined ? 2 : 1;
        if (t->path == NORM_PATH_CLUSTER) {
          ot.cluster_size = t->cluster;
          ot.cluster_rows = t->rows;
          ok = plan_cluster(backward, layernorm, M, N, nvec, dtype, ot, p);
        } else {
          ok = plan_rows(backward, layernorm, M, N, nvec, ot, false, p);
        }
        if (ok) break;
        ok = true;  // the entry does not fit this call: fall through to the rules
        p = Plan();
        p.nvec = int(nvec);
      }
      if (!vec_ok) {
        if (backward) {
          plan_generic_bwd(layernorm, M, N, nvec, atomic, o, p);
        } else if (N <= kGrowsFwdMaxElems) {
          plan_generic_fwd(M, N, o, p);
        } else {
          plan_split(false, layernorm, M, N, nvec, false, o, p);
        }
      } else if (atomic || (backward && nvec <= kBwdRowsMaxVecs)) {
        ok = plan_rows(backward, layernorm, M, N, nvec, o, atomic, p);
      } else if (!backward && nvec <= kFwdRowsMaxVecs &&
                 plan_rows(false, layernorm, M, N, nvec, o, false, p)) {
        // one workgroup holds the row
      } else if (!backward && nvec <= kFwdRowsMaxVecs && (o.lanes_per_row || o.vecs_per_lane)) {
        ok = false;  // the mapping asked for does not cover the row
      } else if (backward && nvec <= kBwdRowsLdsMaxVecs && !o.lanes_per_row &&
                 !o.vecs_per_lane && plan_rows(true, layernorm, M, N, nvec, o, false, p)) {
        // a 1024-lane mapping with LDS partials covers the row
      } else if (!backward && nvec <= kFwdRowsWideMaxVecs && !o.lanes_per_row &&
                 !o.vecs_per_lane && plan_rows(false, layernorm, M, N, nvec, o, false, p)) {
        // a 12- or 16-vector mapping covers the row
      } else if (!plan_cluster(backward, layernorm, M, N, nvec, dtype, o, p)) {
        if (backward || !plan_rows(false, layernorm, M, N, nvec, o, false, p)) {
          p = Plan();
          p.nvec = int(nvec);
          plan_split(backward, layernorm, M, N, nvec, true, o, p);
        }
      }
      break;
    case NORM_PATH_ROWS:
      ok = vec_ok && plan_rows(backward, layernorm, M, N, nvec, o, atomic, p);
      break;
    case NORM_PATH_CLUSTER:
      ok = vec_ok && !atomic && plan_cluster(backward, layernorm, M, N, nvec, dtype, o, p);
      break;
    case NORM_PATH_SPLIT:
      // the backward's sliced passes over elements are its GENERIC plan
      ok = vec_ok || !backward;
      if (ok) plan_split(backward, layernorm, M, N, nvec, vec_ok, o, p);
      break;
    case NORM_PATH_GENERIC:
      if (backward) {
        plan_generic_bwd(layernorm, M, N, nvec, atomic, o, p);
      } else {
        plan_generic_fwd(M, N, o, p);
      }
      break;
  }
  if (!ok) return NORM_ERR_BAD_OPTION;
  if (p.path != NORM_PATH_ROWS && p.path != NORM_PATH_CLUSTER &&
      (o.lanes_per_row || o.vecs_per_lane))
    return NORM_ERR_BAD_OPTION;
  if (p.path != NORM_PATH_CLUSTER && (o.cluster_size || o.cluster_rows)) return NORM_ERR_BAD_OPTION;
  if (p.path != NORM_PATH_ROWS) p.pipelined = false;
  if (atomic && p.path != NORM_PATH_ROWS) return NORM_ERR_BAD_OPTION;

  p.ws_need = p.ws_bytes;
  if (p.path == NORM_PATH_CLUSTER) {
    Plan f;
    make_fallback_plan(backward, layernorm, M, N, dtype, &f);
    if (f.ws_bytes > p.ws_need) p.ws_need = f.ws_bytes;
  }
  if (M == 0) p.grid = 0;
  *out = p;
  return NORM_OK;
}

norm_status_t make_fallback_plan(bool backward, bool layernorm, int64_t M, int64_t N, int dtype,
                                 Plan* out) {
  norm_options_t o = {};
  Plan p;
  const int epv = dtype != NORM_DTYPE_F32 ? 8 : 4;
  p.nvec = int(N / epv);
  plan_split(backward, layernorm, M, N, p.nvec, true, o, p);
  if (M == 0) p.grid = 0;
  p.ws_need = p.ws_bytes;
  *out = p;
  return NORM_OK;
}

norm_status_t make_fwd_plan_without_workspace(bool layernorm, int64_t M, int64_t N, int dtype,
                                              bool aligned16, const norm_options_t* opt,
                                              Plan* out) {
  norm_options_t o = {};
  if (opt) o.grid = opt->grid;
  Plan p;
  const int epv = dtype != NORM_DTYPE_F32 ? 8 : 4;
  const bool vec_ok = aligned16 && (N % epv == 0);
  const int64_t nvec = vec_ok ? N / epv : 0;
  p.nvec = int(nvec);
  if (!(vec_ok && nvec <= kFwdRowsWideMaxVecs && plan_rows(false, layernorm, M, N, nvec, o, false, p))) {
    p = Plan();
    p.nvec = int(nvec);
    plan_generic_fwd(M, N, o, p);
  }
  if (M == 0) p.grid = 0;
  p.ws_need = p.ws_bytes;
  *out = p;
  return NORM_OK;
}

size_t workspace_bytes(bool backward, int64_t M, int64_t N, bool layernorm, int dtype,
                       const norm_options_t* opt) {
  size_t best = 0;
  for (int aligned = 0; aligned < 2; ++aligned) {
    Plan p;
    if (make_plan(backward, layernorm, M, N, dtype, aligned != 0, opt, &p) == NORM_OK &&
        p.ws_need > best)
      best = p.ws_need;
  }
  return best;
}

}  // namespace rownorm
