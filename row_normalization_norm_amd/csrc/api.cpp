// C ABI of the row-normalization library (declared in include/rownorm.h).
//
// Every argument is checked on the host before any HIP call, so an invalid call
// returns its status with nothing enqueued.  Valid calls plan the mapping (plan.cpp)
// and enqueue the kernels on the caller's stream; nothing here synchronises,
// allocates device memory, or keeps a pointer past the call.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <random>

#include "../../include/rownorm.h"
#include "launch.h"
#include "plan.h"

namespace rownorm {

// Per-(kind, type pair) launchers, one translation unit each (TypeCombo in launch.h).
#define RN_DECL_TU(K, T)                                                                  \
  hipError_t launch_fwd_rows_k##K##_t##T(int, int, const FwdArgs&, int, bool, hipStream_t); \
  hipError_t launch_bwd_rows_k##K##_t##T(int, int, const BwdArgs&, int, bool, hipStream_t); \
  hipError_t launch_fwd_cluster_k##K##_t##T(int, int, int, const FwdArgs&, const ClusterArgs&, \
                                            int, hipStream_t);                             \
  hipError_t launch_bwd_cluster_k##K##_t##T(int, int, int, const BwdArgs&, const ClusterArgs&, \
                                            int, hipStream_t);                             \
  int occupancy_fwd_cluster_k##K##_t##T(int, int, int, bool);                              \
  int occupancy_bwd_cluster_k##K##_t##T(int, int, int, bool);                              \
  hipError_t launch_fwd_grows_k##K##_t##T(int, const FwdArgs&, int, hipStream_t);          \
  hipError_t launch_bwd_grows_k##K##_t##T(int, const BwdArgs&, int, hipStream_t);
RN_DECL_TU(0, 0) RN_DECL_TU(0, 1) RN_DECL_TU(0, 2) RN_DECL_TU(0, 3) RN_DECL_TU(0, 4)
RN_DECL_TU(1, 0) RN_DECL_TU(1, 1) RN_DECL_TU(1, 2) RN_DECL_TU(1, 3) RN_DECL_TU(1, 4)
#undef RN_DECL_TU

#define RN_TABLE(PFX)                                                      \
  {                                                                        \
    {PFX##_k0_t0, PFX##_k0_t1, PFX##_k0_t2, PFX##_k0_t3, PFX##_k0_t4}, {   \
      PFX##_k1_t0, PFX##_k1_t1, PFX##_k1_t2, PFX##_k1_t3, PFX##_k1_t4      \
    }                                                                      \
  }

namespace {
using FwdRowsFn = hipError_t (*)(int, int, const FwdArgs&, int, bool, hipStream_t);
using BwdRowsFn = hipError_t (*)(int, int, const BwdArgs&, int, bool, hipStream_t);
using FwdClusterFn = hipError_t (*)(int, int, int, const FwdArgs&, const ClusterArgs&, int,
                                    hipStream_t);
using BwdClusterFn = hipError_t (*)(int, int, int, const BwdArgs&, const ClusterArgs&, int,
                                    hipStream_t);
using OccFn = int (*)(int, int, int, bool);
using FwdGrowsFn = hipError_t (*)(int, const FwdArgs&, int, hipStream_t);
using BwdGrowsFn = hipError_t (*)(int, const BwdArgs&, int, hipStream_t);
const FwdGrowsFn kFwdGrows[2][kNumTypeCombos] = RN_TABLE(launch_fwd_grows);
const BwdGrowsFn kBwdGrows[2][kNumTypeCombos] = RN_TABLE(launch_bwd_grows);
const FwdRowsFn kFwdRows[2][kNumTypeCombos] = RN_TABLE(launch_fwd_rows);
const BwdRowsFn kBwdRows[2][kNumTypeCombos] = RN_TABLE(launch_bwd_rows);
const FwdClusterFn kFwdCluster[2][kNumTypeCombos] = RN_TABLE(launch_fwd_cluster);
const BwdClusterFn kBwdCluster[2][kNumTypeCombos] = RN_TABLE(launch_bwd_cluster);
const OccFn kFwdOcc[2][kNumTypeCombos] = RN_TABLE(occupancy_fwd_cluster);
const OccFn kBwdOcc[2][kNumTypeCombos] = RN_TABLE(occupancy_bwd_cluster);
}  // namespace
#undef RN_TABLE

hipError_t launch_fwd_rows(int kind, int tc, int lpr, int vpl, const FwdArgs& a, int grid,
                           bool pipe, hipStream_t s) {
  return kFwdRows[kind][tc](lpr, vpl, a, grid, pipe, s);
}
hipError_t launch_fwd_grows(int kind, int tc, int epl, const FwdArgs& a, int grid,
                            hipStream_t s) {
  return kFwdGrows[kind][tc](epl, a, grid, s);
}
hipError_t launch_bwd_grows(int kind, int tc, int epl, const BwdArgs& a, int grid,
                            hipStream_t s) {
  return kBwdGrows[kind][tc](epl, a, grid, s);
}
hipError_t launch_bwd_rows(int kind, int tc, int lpr, int vpl, const BwdArgs& a, int grid,
                           bool pipe, hipStream_t s) {
  return kBwdRows[kind][tc](lpr, vpl, a, grid, pipe, s);
}
hipError_t launch_fwd_cluster(int kind, int tc, int t, int vpl, int rows, const FwdArgs& a,
                              const ClusterArgs& c, int grid, hipStream_t s) {
  return kFwdCluster[kind][tc](t, vpl, rows, a, c, grid, s);
}
hipError_t launch_bwd_cluster(int kind, int tc, int t, int vpl, int rows, const BwdArgs& a,
                              const ClusterArgs& c, int grid, hipStream_t s) {
  return kBwdCluster[kind][tc](t, vpl, rows, a, c, grid, s);
}
int occupancy_fwd_cluster(int kind, int tc, int t, int vpl, int rows, bool add) {
  return kFwdOcc[kind][tc](t, vpl, rows, add);
}
int occupancy_bwd_cluster(int kind, int tc, int t, int vpl, int rows, bool add) {
  return kBwdOcc[kind][tc](t, vpl, rows, add);
}

// The public dtype code: the activation type in the low byte, optionally the parameter
// type + 1 in the next byte (0: the activation type), see rownorm.h.
struct DtypeInfo {
  int x = -1;   // activation type (norm_dtype_t)
  int p = -1;   // parameter type
  int tc = -1;  // TypeCombo
};

DtypeInfo decode_dtype(norm_dtype_t code) {
  DtypeInfo d;
  const uint32_t c = static_cast<uint32_t>(code);
  if (c >> 16) return d;
  const int x = int(c & 0xFFu), pc = int((c >> 8) & 0xFFu);
  const int p = pc ? pc - 1 : x;
  const bool x_ok = x == NORM_DTYPE_F32 || x == NORM_DTYPE_BF16 || x == NORM_DTYPE_F16;
  if (!x_ok) return d;
  int tc = -1;
  if (p == x) {
    tc = x == NORM_DTYPE_F32 ? kTcF32 : x == NORM_DTYPE_BF16 ? kTcBF16 : kTcF16;
  } else if (p == NORM_DTYPE_F32 && x == NORM_DTYPE_BF16) {
    tc = kTcBF16F32;
  } else if (p == NORM_DTYPE_F32 && x == NORM_DTYPE_F16) {
    tc = kTcF16F32;
  }
  if (tc < 0) return d;
  d.x = x;
  d.p = p;
  d.tc = tc;
  return d;
}

uintptr_t elem_bytes(int t) { return t == NORM_DTYPE_F32 ? 4 : 2; }

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

norm_status_t check_shape_dtype(int64_t M, int64_t N, norm_dtype_t dtype) {
  if (decode_dtype(dtype).tc < 0) return NORM_ERR_BAD_DTYPE;
  if (M < 0 || N < 1 || N > INT32_MAX) return NORM_ERR_BAD_SHAPE;
  // Keep M*N*16 (the largest byte offset any kernel forms) within int64.
  if (M > 0 && M > (INT64_MAX / 16) / N) return NORM_ERR_BAD_SHAPE;
  return NORM_OK;
}

// NORM_OK, or NORM_ERR_HIP for a failed HIP call; with ROWNORM_DEBUG set in the
// environment the HIP error is also printed to stderr.
norm_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return NORM_OK;
  if (std::getenv("ROWNORM_DEBUG"))
    std::fprintf(stderr, "rownorm: HIP error %d (%s)\n", int(e), hipGetErrorString(e));
  return NORM_ERR_HIP;
}

struct EventScope {
  const norm_options_t* opt;
  hipStream_t stream;
  hipError_t start() const {
    return (opt && opt->ev_start) ? hipEventRecord(opt->ev_start, stream) : hipSuccess;
  }
  hipError_t stop() const {
    return (opt && opt->ev_stop) ? hipEventRecord(opt->ev_stop, stream) : hipSuccess;
  }
};

}  // namespace

// Workgroups of a cluster kernel the current device can hold at once (0 if unknown).
// Cached per (device, direction, kind, type pair, fused add, threads, vectors, rows per
// step).
int cluster_capacity(bool backward, int kind, int tc, bool add, int t, int vpl, int rows) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  static std::atomic<int> cus[64];
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  // occupancy depends only on the kernel and the device's per-CU limits
  static std::mutex mu;
  // [dev][bwd][kind][type pair][add][t: 256/512/1024][vpl: 1/2/4][rows per step: 1/2]
  static int cache[64][2][2][kNumTypeCombos][2][3][3][2];
  const int ti = t == 256 ? 0 : t == 512 ? 1 : 2;
  const int vi = vpl == 1 ? 0 : vpl == 2 ? 1 : 2;
  int occ;
  {
    std::lock_guard<std::mutex> lock(mu);
    const int ri = rows == 1 ? 0 : 1;
    occ = cache[dev][backward][kind][tc][add][ti][vi][ri];
    if (occ == 0) {
      occ = backward ? occupancy_bwd_cluster(kind, tc, t, vpl, rows, add)
                     : occupancy_fwd_cluster(kind, tc, t, vpl, rows, add);
      cache[dev][backward][kind][tc][add][ti][vi][ri] = occ > 0 ? occ : -1;
    }
  }
  return occ > 0 ? occ * n : 0;
}

// Fit a CLUSTER plan to the device: clamp the number of clusters to what can be
// co-resident (fewer clusters also means fewer dgamma/dbeta partial rows, so the
// workspace the plan sized still suffices).  Returns false when not even one cluster
// fits; the caller then takes the fallback plan.
bool fit_cluster(bool backward, int kind, int tc, bool add, Plan& p) {
  const int cap = cluster_capacity(backward, kind, tc, add, p.lpr, p.vpl, p.rows_per_step);
  if (cap < p.cluster) return false;
  if (p.grid > cap) {
    int ncl = cap / p.cluster;
    if (ncl >= 8) ncl -= ncl % 8;
    p.nclusters = ncl;
    p.grid = ncl * p.cluster;
    if (backward) p.partial_rows = ncl;
  }
  return true;
}

namespace {

// The SplitMix64 output function (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014), a bijection that spreads the epochs, which count up, over
// all 64 bits of the kernels' tag base.
uint64_t tag_base(uint64_t epoch) {
  uint64_t z = epoch;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

ClusterArgs cluster_args(const Plan& p, char* ws, const norm_options_t* opt, uint64_t epoch) {
  ClusterArgs c;
  c.tag_base = tag_base(epoch);
  c.C = p.cluster;
  c.nclusters = p.nclusters;
  c.slice_vecs = p.slice_vecs;
  c.rows_per_step = p.rows_per_step;
  const int wait = opt ? opt->cluster_wait : 0;
  c.spin_limit = wait > 0 ? uint32_t(wait) : wait < 0 ? 0u : kSpinLimit;
  c.xchg = reinterpret_cast<unsigned long long*>(ws + p.off_xchg);
  return c;
}

// Zero the exchange slots before a cluster launch.  A fill kernel rather than a memset,
// so the call stays safe to capture in a graph.
hipError_t clear_exchange(const Plan& p, char* ws, hipStream_t s) {
  return launch_zero(reinterpret_cast<float*>(ws + p.off_xchg), nullptr,
                     int32_t(p.xchg_bytes / 4), s);
}

// Epochs of split-row launches: odd (0 is the epoch of captured calls), distinct within
// the process, and starting from a random point so that words another process left in
// reused memory do not share them.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{[] {
    uint64_t seed = static_cast<uint64_t>(
        std::chrono::steady_clock::now().time_since_epoch().count());
    try {
      std::random_device rd;
      seed ^= (static_cast<uint64_t>(rd()) << 32) ^ rd();
    } catch (...) {
    }
    return seed;
  }()};
  return (counter.fetch_add(1, std::memory_order_relaxed) << 1) | 1u;
}

// The exchange of one split-row launch.  A call outside graph capture gets a fresh
// epoch, which the tags of its words carry, so the words earlier calls left in the
// workspace (and whatever else it holds) do not match and nothing needs clearing.  A
// captured call would replay one epoch, so it takes epoch 0 and zeroes the slots with a
// fill kernel that is captured with it.
hipError_t prepare_exchange(const Plan& p, char* ws, hipStream_t s, uint64_t* epoch) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    *epoch = 0;
    return clear_exchange(p, ws, s);
  }
  *epoch = next_epoch();
  return hipSuccess;
}

// ------------------------------------------------------------- static scratch
// Device memory for norm_ln_bwd_noalloc, for callers that cannot allocate: the
// dgamma/dbeta partial rows and, for split rows, the exchange words, which the
// backward's kernels otherwise take from the caller's workspace.  Every device the
// library runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address scratch_address()
// obtains from the runtime is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The current device's copy of `scratch`, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<void*> addr[64];
  static std::mutex mu;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

norm_status_t check_workspace(const Plan& p, void* workspace, size_t given) {
  if (p.ws_need == 0) return NORM_OK;
  if (!workspace) return NORM_ERR_NULL_PTR;
  if (!aligned(workspace, 16)) return NORM_ERR_MISALIGNED;
  if (given < p.ws_need) return NORM_ERR_WORKSPACE_TOO_SMALL;
  return NORM_OK;
}

// fused: the residual-add entry points (res and sum required when M > 0).
norm_status_t fwd_impl(bool ln, const void* x, const void* gamma, const void* beta, void* y,
                       float* mean, float* rstd, int64_t M, int64_t N, float eps,
                       norm_dtype_t dtype, void* workspace, size_t workspace_bytes_given,
                       hipStream_t stream, const norm_options_t* opt, bool fused = false,
                       const void* res = nullptr, void* sum = nullptr) {
  norm_status_t st = check_shape_dtype(M, N, dtype);
  if (st != NORM_OK) return st;
  if (!gamma || (ln && !beta)) return NORM_ERR_NULL_PTR;
  if (M > 0 && (!x || !y)) return NORM_ERR_NULL_PTR;
  if (fused && M > 0 && (!res || !sum)) return NORM_ERR_NULL_PTR;
  if (!std::isfinite(eps) || eps < 0.0f) return NORM_ERR_BAD_EPS;
  const DtypeInfo dt = decode_dtype(dtype);
  const uintptr_t es = elem_bytes(dt.x), ps = elem_bytes(dt.p);
  if (!aligned(x, es) || !aligned(y, es) || !aligned(gamma, ps) || !aligned(beta, ps) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(res, es) || !aligned(sum, es))
    return NORM_ERR_MISALIGNED;
  const bool a16 = aligned(x, 16) && aligned(y, 16) && aligned(gamma, 16) && aligned(beta, 16) &&
                   aligned(res, 16) && aligned(sum, 16);

  Plan p;
  st = make_plan(false, ln, M, N, dt.x, a16, opt, &p);
  if (st != NORM_OK) return st;
  // The forward's workspace is optional: only split rows (their exchange words) and the
  // sliced passes (their per-row tables) use one.  Given none, or too little, the call
  // takes a plan that needs none, unless one of those paths was asked for explicitly.
  const bool forced_ws = opt && (opt->path == NORM_PATH_CLUSTER || opt->path == NORM_PATH_SPLIT);
  if (p.ws_need > 0 && !forced_ws &&
      (!workspace || workspace_bytes_given < p.ws_need)) {
    st = make_fwd_plan_without_workspace(ln, M, N, dt.x, a16, opt, &p);
    if (st != NORM_OK) return st;
  }
  st = check_workspace(p, workspace, workspace_bytes_given);
  if (st != NORM_OK) return st;
  if (M == 0) return NORM_OK;

  FwdArgs a;
  a.x = x;
  a.gamma = gamma;
  a.beta = beta;
  a.y = y;
  a.mean = mean;
  a.rstd = rstd;
  a.M = M;
  a.N = int32_t(N);
  a.nvec = p.nvec;
  a.eps = eps;
  a.inv_n = 1.0f / float(N);
  a.groups = p.groups;
  a.res = fused ? res : nullptr;
  a.sum = fused ? sum : nullptr;
  a.static_end = p.groups;
  a.persistent = 0;
  a.rowp = nullptr;
  a.rowtab = nullptr;
  a.rows_per_block = 0;
  a.slices = 0;

  const int kind = ln ? 1 : 0;
  EventScope ev{opt, stream};
  char* ws = static_cast<char*>(workspace);
  if (p.path == NORM_PATH_CLUSTER && !fit_cluster(false, kind, dt.tc, fused, p)) {
    make_fallback_plan(false, ln, M, N, dt.x, &p);
  }
  hipError_t e = hipSuccess;
  uint64_t epoch = 0;
  if (p.path == NORM_PATH_CLUSTER) {
    e = prepare_exchange(p, ws, stream, &epoch);
    if (e != hipSuccess) return hip_status(e);
  }
  if ((e = ev.start()) != hipSuccess) return hip_status(e);
  switch (p.path) {
    case NORM_PATH_ROWS:
      e = launch_fwd_rows(kind, dt.tc, p.lpr, p.vpl, a, p.grid, p.pipelined, stream);
      break;
    case NORM_PATH_CLUSTER:
      e = launch_fwd_cluster(kind, dt.tc, p.lpr, p.vpl, p.rows_per_step, a,
                             cluster_args(p, ws, opt, epoch),
                             p.grid, stream);
      break;
    case NORM_PATH_SPLIT:
      a.rowtab = reinterpret_cast<float*>(ws + p.off_rowc);
      a.rowp = reinterpret_cast<float*>(ws + p.off_rowp);
      a.rows_per_block = p.rows_per_block;
      a.slices = p.slices;
      e = launch_fwd_split(kind, dt.tc, p.vec, a, p.slices, int(p.row_blocks), p.grid, stream);
      break;
    default:
      e = p.vpl > 0 ? launch_fwd_grows(kind, dt.tc, p.vpl, a, p.grid, stream)
                    : launch_fwd_generic(kind, dt.tc, a, p.grid, stream);
  }
  if (e != hipSuccess) return hip_status(e);
  return hip_status(ev.stop());
}

// dres: the residual-add entry points' gradient arriving at the sum (may be NULL).
// use_scratch: the workspace is the library's static scratch array (the entry point
// that allocates nothing); the workspace arguments are then ignored.
norm_status_t bwd_impl(bool ln, const void* dy, const void* x, const void* gamma,
                       const float* mean, const float* rstd, void* dx, float* dgamma,
                       float* dbeta, int64_t M, int64_t N, norm_dtype_t dtype, void* workspace,
                       size_t workspace_bytes_given, hipStream_t stream,
                       const norm_options_t* opt, const void* dres = nullptr,
                       bool use_scratch = false) {
  norm_status_t st = check_shape_dtype(M, N, dtype);
  if (st != NORM_OK) return st;
  if (!gamma || !dgamma || (ln && !dbeta)) return NORM_ERR_NULL_PTR;
  if (M > 0 && (!dy || !x || !rstd || !dx || (ln && !mean))) return NORM_ERR_NULL_PTR;
  const DtypeInfo dt = decode_dtype(dtype);
  const uintptr_t es = elem_bytes(dt.x), ps = elem_bytes(dt.p);
  if (!aligned(dy, es) || !aligned(x, es) || !aligned(gamma, ps) || !aligned(dx, es) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dgamma, 4) || !aligned(dbeta, 4) ||
      !aligned(dres, es))
    return NORM_ERR_MISALIGNED;
  const bool a16 = aligned(dy, 16) && aligned(x, 16) && aligned(gamma, 16) && aligned(dx, 16) &&
                   aligned(dres, 16);

  Plan p;
  st = make_plan(true, ln, M, N, dt.x, a16, opt, &p);
  if (st != NORM_OK) return st;
  if (use_scratch) {
    // the last check before the first HIP call
    if (p.ws_need > kScratchBytes) return NORM_ERR_SCRATCH_TOO_SMALL;
    workspace = nullptr;
    workspace_bytes_given = kScratchBytes;
    if (p.ws_need > 0) {
      hipError_t e = scratch_address(&workspace);
      if (e != hipSuccess) return hip_status(e);
    }
  }
  st = check_workspace(p, workspace, workspace_bytes_given);
  if (st != NORM_OK) return st;

  const int kind = ln ? 1 : 0;
  const int mode = opt ? opt->dgamma_mode : NORM_DGAMMA_TWO_STAGE;
  float* const db = ln ? dbeta : nullptr;

  if (M == 0) {  // a sum over no rows
    return hip_status(launch_zero(dgamma, db, int32_t(N), stream));
  }

  char* ws = static_cast<char*>(workspace);
  if (p.path == NORM_PATH_CLUSTER && !fit_cluster(true, kind, dt.tc, dres != nullptr, p)) {
    make_fallback_plan(true, ln, M, N, dt.x, &p);
  }
  BwdArgs a;
  a.dy = dy;
  a.x = x;
  a.gamma = gamma;
  a.mean = mean;
  a.rstd = rstd;
  a.dx = dx;
  a.part_g = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_part_g) : nullptr;
  a.part_b = (p.ws_bytes && ln) ? reinterpret_cast<float*>(ws + p.off_part_b) : nullptr;
  a.dgamma = dgamma;
  a.dbeta = db;
  // the split paths: a per-row pass, then a column-sliced pass (GENERIC rows too long for
  // the register-resident scalar kernel, whose plan has vpl = 0)
  const bool two_pass =
      p.path == NORM_PATH_SPLIT || (p.path == NORM_PATH_GENERIC && p.vpl == 0);
  a.rowc = two_pass ? reinterpret_cast<float*>(ws + p.off_rowc) : nullptr;
  a.rowp = two_pass ? reinterpret_cast<float*>(ws + p.off_rowp) : nullptr;
  a.slices = two_pass ? p.slices : 0;
  a.M = M;
  a.N = int32_t(N);
  a.nvec = p.nvec;
  a.inv_n = 1.0f / float(N);
  a.mode = mode;
  a.groups = p.groups;
  a.rows_per_block = p.col_rows_per_block;
  a.dres = dres;

  EventScope ev{opt, stream};
  hipError_t e = hipSuccess;
  if (mode != NORM_DGAMMA_TWO_STAGE) {
    e = launch_zero(dgamma, db, int32_t(N), stream);
    if (e != hipSuccess) return hip_status(e);
  }
  uint64_t epoch = 0;
  if (p.path == NORM_PATH_CLUSTER) {
    e = prepare_exchange(p, ws, stream, &epoch);
    if (e != hipSuccess) return hip_status(e);
  }
  if ((e = ev.start()) != hipSuccess) return hip_status(e);
  if (p.path == NORM_PATH_ROWS) {
    e = launch_bwd_rows(kind, dt.tc, p.lpr, p.vpl, a, p.grid, p.pipelined, stream);
  } else if (p.path == NORM_PATH_CLUSTER) {
    e = launch_bwd_cluster(kind, dt.tc, p.lpr, p.vpl, p.rows_per_step, a,
                           cluster_args(p, ws, opt, epoch), p.grid, stream);
  } else if (!two_pass) {
    e = launch_bwd_grows(kind, dt.tc, p.vpl, a, p.grid, stream);
  } else {
    e = launch_bwd_split(kind, dt.tc, p.vec, a, p.slices, int(p.row_blocks), p.rows_per_block,
                         int(p.partial_rows), p.col_rows_per_block, p.grid, stream);
  }
  if (e != hipSuccess) return hip_status(e);
  if ((e = ev.stop()) != hipSuccess) return hip_status(e);
  if (mode == NORM_DGAMMA_TWO_STAGE) {
    e = launch_colreduce(a.part_g, a.part_b, p.partial_rows, int32_t(N), dgamma, db, stream);
  }
  return hip_status(e);
}

template <typename F>
norm_status_t guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return NORM_ERR_HIP;
  }
}

}  // namespace
}  // namespace rownorm

using rownorm::bwd_impl;
using rownorm::fwd_impl;
using rownorm::guarded;

extern "C" {

norm_status_t norm_rms_fwd(const void* x, const void* gamma, void* y, float* rstd, int64_t M,
                           int64_t N, float eps, norm_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return guarded([&] {
    return fwd_impl(false, x, gamma, nullptr, y, nullptr, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, nullptr);
  });
}

norm_status_t norm_ln_fwd(const void* x, const void* gamma, const void* beta, void* y,
                          float* mean, float* rstd, int64_t M, int64_t N, float eps,
                          norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return guarded([&] {
    return fwd_impl(true, x, gamma, beta, y, mean, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, nullptr);
  });
}

norm_status_t norm_rms_fwd_ex(const void* x, const void* gamma, void* y, float* rstd, int64_t M,
                              int64_t N, float eps, norm_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream,
                              const norm_options_t* opt) {
  return guarded([&] {
    return fwd_impl(false, x, gamma, nullptr, y, nullptr, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, opt);
  });
}

norm_status_t norm_ln_fwd_ex(const void* x, const void* gamma, const void* beta, void* y,
                             float* mean, float* rstd, int64_t M, int64_t N, float eps,
                             norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, const norm_options_t* opt) {
  return guarded([&] {
    return fwd_impl(true, x, gamma, beta, y, mean, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, opt);
  });
}

size_t norm_fwd_workspace_size(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype) {
  return norm_fwd_workspace_size_ex(M, N, is_layernorm, dtype, nullptr);
}

size_t norm_fwd_workspace_size_ex(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype,
                                  const norm_options_t* opt) {
  if (rownorm::check_shape_dtype(M, N, dtype) != NORM_OK) return 0;
  return rownorm::workspace_bytes(false, M, N, is_layernorm != 0, rownorm::decode_dtype(dtype).x,
                                  opt);
}

size_t norm_bwd_workspace_size(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype) {
  return norm_bwd_workspace_size_ex(M, N, is_layernorm, dtype, nullptr);
}

size_t norm_bwd_workspace_size_ex(int64_t M, int64_t N, int is_layernorm, norm_dtype_t dtype,
                                  const norm_options_t* opt) {
  if (rownorm::check_shape_dtype(M, N, dtype) != NORM_OK) return 0;
  return rownorm::workspace_bytes(true, M, N, is_layernorm != 0, rownorm::decode_dtype(dtype).x,
                                  opt);
}

norm_status_t norm_rms_bwd(const void* dy, const void* x, const void* gamma, const float* rstd,
                           void* dx, float* dgamma, int64_t M, int64_t N, norm_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&] {
    return bwd_impl(false, dy, x, gamma, nullptr, rstd, dx, dgamma, nullptr, M, N, dtype,
                    workspace, workspace_bytes, stream, nullptr);
  });
}

norm_status_t norm_ln_bwd(const void* dy, const void* x, const void* gamma, const float* mean,
                          const float* rstd, void* dx, float* dgamma, float* dbeta, int64_t M,
                          int64_t N, norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return guarded([&] {
    return bwd_impl(true, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, workspace,
                    workspace_bytes, stream, nullptr);
  });
}

norm_status_t norm_rms_bwd_ex(const void* dy, const void* x, const void* gamma,
                              const float* rstd, void* dx, float* dgamma, int64_t M, int64_t N,
                              norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const norm_options_t* opt) {
  return guarded([&] {
    return bwd_impl(false, dy, x, gamma, nullptr, rstd, dx, dgamma, nullptr, M, N, dtype,
                    workspace, workspace_bytes, stream, opt);
  });
}

norm_status_t norm_ln_bwd_ex(const void* dy, const void* x, const void* gamma,
                             const float* mean, const float* rstd, void* dx, float* dgamma,
                             float* dbeta, int64_t M, int64_t N, norm_dtype_t dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             const norm_options_t* opt) {
  return guarded([&] {
    return bwd_impl(true, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, workspace,
                    workspace_bytes, stream, opt);
  });
}

norm_status_t norm_ln_bwd_noalloc(const void* dy, const void* x, const void* gamma,
                                  const float* mean, const float* rstd, void* dx, float* dgamma,
                                  float* dbeta, int64_t M, int64_t N, norm_dtype_t dtype,
                                  hipStream_t stream) {
  return guarded([&] {
    return bwd_impl(true, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, nullptr, 0,
                    stream, nullptr, nullptr, true);
  });
}

norm_status_t norm_rms_fwd_add(const void* x, const void* residual, const void* gamma, void* y,
                               void* sum, float* rstd, int64_t M, int64_t N, float eps,
                               norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, const norm_options_t* opt) {
  return guarded([&] {
    return fwd_impl(false, x, gamma, nullptr, y, nullptr, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, opt, true, residual, sum);
  });
}

norm_status_t norm_ln_fwd_add(const void* x, const void* residual, const void* gamma,
                              const void* beta, void* y, void* sum, float* mean, float* rstd,
                              int64_t M, int64_t N, float eps, norm_dtype_t dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              const norm_options_t* opt) {
  return guarded([&] {
    return fwd_impl(true, x, gamma, beta, y, mean, rstd, M, N, eps, dtype, workspace,
                    workspace_bytes, stream, opt, true, residual, sum);
  });
}

norm_status_t norm_rms_bwd_add(const void* dy, const void* sum, const void* gamma,
                               const float* rstd, const void* dsum, void* dx, float* dgamma,
                               int64_t M, int64_t N, norm_dtype_t dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream,
                               const norm_options_t* opt) {
  return guarded([&] {
    return bwd_impl(false, dy, sum, gamma, nullptr, rstd, dx, dgamma, nullptr, M, N, dtype,
                    workspace, workspace_bytes, stream, opt, dsum);
  });
}

norm_status_t norm_ln_bwd_add(const void* dy, const void* sum, const void* gamma,
                              const float* mean, const float* rstd, const void* dsum, void* dx,
                              float* dgamma, float* dbeta, int64_t M, int64_t N,
                              norm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const norm_options_t* opt) {
  return guarded([&] {
    return bwd_impl(true, dy, sum, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, workspace,
                    workspace_bytes, stream, opt, dsum);
  });
}

norm_status_t norm_plan(int is_backward, int is_layernorm, int64_t M, int64_t N,
                        norm_dtype_t dtype, int aligned16, const norm_options_t* opt,
                        norm_plan_info_t* info) {
  if (!info) return NORM_ERR_NULL_PTR;
  norm_status_t st = rownorm::check_shape_dtype(M, N, dtype);
  if (st != NORM_OK) return st;
  rownorm::Plan p;
  st = rownorm::make_plan(is_backward != 0, is_layernorm != 0, M, N, rownorm::decode_dtype(dtype).x,
                          aligned16 != 0, opt, &p);
  if (st != NORM_OK) return st;
  info->path = p.path;
  info->lanes_per_row = p.lpr;
  info->vecs_per_lane = p.vpl;
  info->block = p.block;
  // the sliced passes report their (slice, row block) grid
  info->grid = p.slices ? int(p.slices * p.row_blocks) : p.grid;
  info->partial_rows = int(p.partial_rows);
  info->cluster_size = p.cluster;
  info->cluster_rows = p.rows_per_step;
  info->workspace_bytes = p.ws_need;
  info->pipelined = p.pipelined ? 1 : 0;
  return NORM_OK;
}

int norm_cluster_resident(int is_backward, int is_layernorm, int64_t M, int64_t N,
                          norm_dtype_t dtype, const norm_options_t* opt) {
  if (rownorm::check_shape_dtype(M, N, dtype) != NORM_OK) return -1;
  const rownorm::DtypeInfo dt = rownorm::decode_dtype(dtype);
  rownorm::Plan p;
  if (rownorm::make_plan(is_backward != 0, is_layernorm != 0, M, N, dt.x, true, opt, &p) != NORM_OK)
    return -1;
  if (p.path != NORM_PATH_CLUSTER) return 0;
  return rownorm::fit_cluster(is_backward != 0, is_layernorm ? 1 : 0, dt.tc, false, p) ? 1 : 0;
}

norm_status_t norm_stream_reference(int kind, const void* a, const void* b, void* dst, int64_t n,
                                    hipStream_t stream) {
  return rownorm::guarded([&] {
    if (kind != 0 && kind != 1) return NORM_ERR_BAD_OPTION;
    if (n < 0) return NORM_ERR_BAD_SHAPE;
    if (n == 0) return NORM_OK;
    if (!a || !dst || (kind == 1 && !b)) return NORM_ERR_NULL_PTR;
    if (!rownorm::aligned(a, 16) || !rownorm::aligned(dst, 16) ||
        (kind == 1 && !rownorm::aligned(b, 16)))
      return NORM_ERR_MISALIGNED;
    return rownorm::hip_status(
        rownorm::launch_stream_reference(kind == 1, a, b, dst, n, stream));
  });
}

const char* norm_status_string(norm_status_t s) {
  switch (s) {
    case NORM_OK: return "ok";
    case NORM_ERR_NULL_PTR: return "a required pointer is NULL";
    case NORM_ERR_BAD_SHAPE: return "bad shape (need M >= 0, 1 <= N <= 2^31-1)";
    case NORM_ERR_BAD_DTYPE: return "bad dtype";
    case NORM_ERR_BAD_EPS: return "eps must be finite and >= 0";
    case NORM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NORM_ERR_HIP: return "HIP runtime error";
    case NORM_ERR_MISALIGNED: return "pointer not aligned to its element size";
    case NORM_ERR_BAD_OPTION: return "bad option";
    case NORM_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more than the library's 32 MiB static scratch";
  }
  return "unknown status";
}

}  // extern "C"
