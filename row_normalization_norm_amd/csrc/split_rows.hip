// Rows too long for one workgroup's registers or a cluster (and rows that are not whole
// 16-byte vectors, past the register-resident scalar kernels): each row is cut into
// column slices of kSliceBlock lanes x V units (16-byte vectors, or single elements),
// and every pass runs on a (slice, row block) grid, so a single row still spreads over
// the whole chip.  The passes meet through small per-(row, slice) tables in the
// workspace:
//
//  forward   slicestats -- per slice of a row: RMSNorm the sum of squares; LayerNorm the
//                          sum and the sum of squared deviations about the slice's mean
//                          (x, or the residual sum x + res, which this pass writes).
//            rowmerge   -- per row (one wavefront): the slices' terms combined into the
//                          row's statistics; LayerNorm with the parallel form of the
//                          update of Chan, Golub and LeVeque (total mean first, then each
//                          slice's squared deviations plus its count times the squared
//                          offset of its mean), so no mean(x^2) - mean^2 cancellation.
//                          Writes (mean, rstd) to the table and to the caller's buffers.
//            slicenorm  -- y = (x - mean) * rstd * gamma (+ beta) over each slice, x read
//                          a second time (the price of rows this long; a recent read is
//                          often still in the memory-side cache).
//  backward  slicedot   -- per slice: sum of g * xhat and of g, g = dy * gamma.
//            rowmerge   -- per row: c1 = sum g * xhat / N, c2 = sum g / N.
//            colslice   -- dx = rstd * (g - c2 - xhat * c1) from the table; per-column
//                          dgamma/dbeta sums of a block of rows in registers, written as
//                          one partial row per row block (then colreduce_kernel).
//
// The operations are those of the row kernels: the forward of "Fused RMSNorm"
// (aryanashta.me, "What it is") and LayerNorm, the backward of "SOTA normalization
// performance with torch.compile" ("Why Is Peak Vectorization Your New Best Friend?"),
// with the two-stage dgamma/dbeta reduction ("Fused RMSNorm", "Next").  Every sum is
// taken in a fixed order, so results are reproducible bit for bit.
#include <type_traits>

#include "launch.h"
#include "rownorm_dev.h"

namespace rownorm {
namespace {

constexpr int kSW = kSliceBlock / 64;           // wavefronts of a slice workgroup
constexpr int kMergeRows = kMergeBlock / 64;    // rows merged per workgroup

// Sums of K values over the workgroup, the same bits in every thread.  `red` holds
// 2 * K * kSW floats, used alternately by parity, so one barrier per call suffices.
template <int K>
__device__ inline void slice_sum(float (&v)[K], float* red, int& parity) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = group_sum<64>(v[k]);
  const int wave = threadIdx.x >> 6;
  float* buf = red + parity * K * kSW;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) buf[k * kSW + wave] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kSW; ++w) t += buf[k * kSW + w];
    v[k] = t;
  }
  parity ^= 1;
}

// The units (16-byte vectors when VEC, else elements) a lane owns in slice `s`: V runs of
// kSliceBlock consecutive units, so each load instruction of a wavefront is contiguous.
template <int V>
struct SliceLanes {
  int64_t idx[V];
  bool own[V];
  __device__ inline SliceLanes(int64_t s, int64_t units) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      idx[v] = (s * V + v) * kSliceBlock + threadIdx.x;
      own[v] = idx[v] < units;
    }
  }
};

// The parameters (gamma or beta) of a lane's units, unpacked to fp32.
template <typename D, typename P, bool VEC, int V, int EPV>
__device__ inline void load_params(const void* base, const SliceLanes<V>& sl,
                                   float (&out)[V][EPV]) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if constexpr (VEC) {
      Param<D, P> pv;
      if (sl.own[v]) {
        pv.load(base, sl.idx[v]);
      } else {
        pv.clear();
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) out[v][e] = pv.get(e);
    } else {
      out[v][0] = sl.own[v] ? P::scalar(base, sl.idx[v]) : 0.0f;
    }
  }
}

// -------------------------------------------------------------------- slicestats
template <bool LN, typename D, typename P, bool VEC>
__global__ __launch_bounds__(kSliceBlock) void fwd_slicestats_kernel(const FwdArgs a) {
  constexpr int EPV = VEC ? D::kPerVec : 1;
  constexpr int V = VEC ? kSliceVecs : kSliceElems;
  __shared__ float red[2 * kSW];
  int parity = 0;
  const int64_t units = VEC ? a.nvec : a.N;
  const int64_t s = blockIdx.x;
  const SliceLanes<V> sl(s, units);
  const int64_t first = s * V * kSliceBlock;
  const int64_t nu = units - first < V * kSliceBlock ? units - first : V * kSliceBlock;
  const float inv_ns = 1.0f / static_cast<float>(nu * EPV);
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;

  for (int64_t row = r0; row < r1; ++row) {
    float xs[V][EPV];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!sl.own[v]) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) xs[v][e] = 0.0f;
        continue;
      }
      if constexpr (VEC) {
        const int64_t vi = row * a.nvec + sl.idx[v];
        u32x4 xv = ld16(a.x, vi);
        if (a.res) {  // the residual sum, rounded to the activation type, is normalized
          xv = D::add(xv, ld16(a.res, vi));
          st16(a.sum, vi, xv);
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) xs[v][e] = D::get(xv, e);
      } else {
        const int64_t i = row * a.N + sl.idx[v];
        float f = D::scalar(a.x, i);
        if (a.res) {
          f = D::round(f + D::scalar(a.res, i));
          D::put_scalar(a.sum, i, f);
        }
        xs[v][0] = f;
      }
    }
    float t[1] = {0.0f}, q[1] = {0.0f};
    if constexpr (LN) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) t[0] += xs[v][e];
      slice_sum<1>(t, red, parity);
      const float mu = t[0] * inv_ns;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (!sl.own[v]) continue;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float d = xs[v][e] - mu;
          q[0] = fmaf(d, d, q[0]);
        }
      }
      slice_sum<1>(q, red, parity);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) t[0] = fmaf(xs[v][e], xs[v][e], t[0]);
      slice_sum<1>(t, red, parity);
    }
    if (threadIdx.x == 0) {
      float* p = a.rowp + (row * a.slices + s) * 2;
      p[0] = t[0];
      p[1] = q[0];
    }
  }
}

// ---------------------------------------------------------------------- rowmerge
// MODE 0: RMSNorm forward, 1: LayerNorm forward, 2: RMSNorm backward, 3: LayerNorm
// backward.  One wavefront per row: lane l takes slices l, l + 64, ..., then the lanes'
// terms are summed across the wavefront.
template <int MODE>
__global__ __launch_bounds__(kMergeBlock) void rowmerge_kernel(const MergeArgs m) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kMergeRows;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kMergeRows + (threadIdx.x >> 6);
       row < m.M; row += stride) {
    const float* p = m.rowp + row * m.slices * 2;
    float u = 0.0f, w = 0.0f;
    for (int s = lane; s < m.slices; s += 64) {
      u += p[2 * s];
      if constexpr (MODE != 1) w += p[2 * s + 1];
    }
    u = group_sum<64>(u);
    if constexpr (MODE == 1) {
      // squared deviations about the row mean: each slice's own, plus its count times
      // the squared offset of its mean from the row's
      const float mu = u * m.inv_n;
      for (int s = lane; s < m.slices; s += 64) {
        const int64_t left = static_cast<int64_t>(m.N) - static_cast<int64_t>(s) * m.slice_elems;
        const float ns = static_cast<float>(left < m.slice_elems ? left : m.slice_elems);
        const float d = p[2 * s] / ns - mu;
        w += p[2 * s + 1] + ns * d * d;
      }
      w = group_sum<64>(w);
      const float r = rsqrtf(w * m.inv_n + m.eps);
      if (lane == 0) {
        m.out[2 * row] = mu;
        m.out[2 * row + 1] = r;
        if (m.mean) m.mean[row] = mu;
        if (m.rstd) m.rstd[row] = r;
      }
    } else if constexpr (MODE == 0) {
      const float r = rsqrtf(u * m.inv_n + m.eps);
      if (lane == 0) {
        m.out[2 * row] = 0.0f;
        m.out[2 * row + 1] = r;
        if (m.rstd) m.rstd[row] = r;
      }
    } else {
      w = group_sum<64>(w);
      if (lane == 0) {
        m.out[2 * row] = u * m.inv_n;
        m.out[2 * row + 1] = MODE == 3 ? w * m.inv_n : 0.0f;
      }
    }
  }
}

// --------------------------------------------------------------------- slicenorm
template <bool LN, typename D, typename P, bool VEC>
__global__ __launch_bounds__(kSliceBlock) void fwd_slicenorm_kernel(const FwdArgs a) {
  constexpr int EPV = VEC ? D::kPerVec : 1;
  constexpr int V = VEC ? kSliceVecs : kSliceElems;
  const int64_t units = VEC ? a.nvec : a.N;
  const SliceLanes<V> sl(blockIdx.x, units);
  float gam[V][EPV], bet[LN ? V : 1][EPV];
  load_params<D, P, VEC>(a.gamma, sl, gam);
  if constexpr (LN) load_params<D, P, VEC>(a.beta, sl, bet);
  // the normalized value: x, or the residual sum the statistics pass wrote
  const void* src = a.res ? a.sum : a.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;

#pragma unroll 2
  for (int64_t row = r0; row < r1; ++row) {
    const float mu = LN ? a.rowtab[2 * row] : 0.0f;
    const float r = a.rowtab[2 * row + 1];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!sl.own[v]) continue;
      if constexpr (VEC) {
        const int64_t vi = row * a.nvec + sl.idx[v];
        const u32x4 xv = ld16_stream(src, vi);
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float f = D::get(xv, e);
          if constexpr (LN) {
            o[e] = fmaf((f - mu) * r, gam[v][e], bet[v][e]);
          } else {
            o[e] = f * r * gam[v][e];
          }
        }
        st16_stream(a.y, vi, D::pack(o));
      } else {
        const int64_t i = row * a.N + sl.idx[v];
        const float f = D::scalar(src, i);
        float o;
        if constexpr (LN) {
          o = fmaf((f - mu) * r, gam[v][0], bet[v][0]);
        } else {
          o = f * r * gam[v][0];
        }
        D::put_scalar(a.y, i, o);
      }
    }
  }
}

// ---------------------------------------------------------------------- slicedot
template <bool LN, typename D, typename P, bool VEC>
__global__ __launch_bounds__(kSliceBlock) void bwd_slicedot_kernel(const BwdArgs a) {
  constexpr int EPV = VEC ? D::kPerVec : 1;
  constexpr int V = VEC ? kSliceVecs : kSliceElems;
  __shared__ float red[2 * 2 * kSW];
  int parity = 0;
  const int64_t units = VEC ? a.nvec : a.N;
  const int64_t s = blockIdx.x;
  const SliceLanes<V> sl(s, units);
  float gam[V][EPV];
  load_params<D, P, VEC>(a.gamma, sl, gam);
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;

  for (int64_t row = r0; row < r1; ++row) {
    const float r = a.rstd[row];
    const float mu = LN ? a.mean[row] : 0.0f;
    float t[2] = {0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!sl.own[v]) continue;
      if constexpr (VEC) {
        const int64_t vi = row * a.nvec + sl.idx[v];
        const u32x4 xv = ld16(a.x, vi);
        const u32x4 dv = ld16(a.dy, vi);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float xh = (D::get(xv, e) - mu) * r;
          const float g = D::get(dv, e) * gam[v][e];
          t[0] = fmaf(g, xh, t[0]);
          if constexpr (LN) t[1] += g;
        }
      } else {
        const int64_t i = row * a.N + sl.idx[v];
        const float xh = (D::scalar(a.x, i) - mu) * r;
        const float g = D::scalar(a.dy, i) * gam[v][0];
        t[0] = fmaf(g, xh, t[0]);
        if constexpr (LN) t[1] += g;
      }
    }
    slice_sum<2>(t, red, parity);
    if (threadIdx.x == 0) {
      float* p = a.rowp + (row * a.slices + s) * 2;
      p[0] = t[0];
      p[1] = t[1];
    }
  }
}

// --------------------------------------------------------------------- colslice
template <bool LN, typename D, typename P, bool VEC>
__global__ __launch_bounds__(kSliceBlock) void colslice_kernel(const BwdArgs a) {
  constexpr int EPV = VEC ? D::kPerVec : 1;
  constexpr int V = VEC ? kSliceVecs : kSliceElems;
  const int64_t units = VEC ? a.nvec : a.N;
  const SliceLanes<V> sl(blockIdx.x, units);
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.M ? r0 + a.rows_per_block : a.M;

  float gam[V][EPV];
  load_params<D, P, VEC>(a.gamma, sl, gam);

  float accg[V][EPV], accb[LN ? V : 1][EPV];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      accg[v][e] = 0.0f;
      if constexpr (LN) accb[v][e] = 0.0f;
    }
  }

#pragma unroll 2
  for (int64_t row = r0; row < r1; ++row) {
    const float r = a.rstd[row];
    const float mu = LN ? a.mean[row] : 0.0f;
    const float c1 = a.rowc[2 * row];
    const float c2 = a.rowc[2 * row + 1];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!sl.own[v]) continue;
      float xs[EPV], ds[EPV];
      if constexpr (VEC) {
        const int64_t vi = row * a.nvec + sl.idx[v];
        const u32x4 xv = ld16_stream(a.x, vi);
        const u32x4 dv = ld16_stream(a.dy, vi);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          xs[e] = D::get(xv, e);
          ds[e] = D::get(dv, e);
        }
      } else {
        const int64_t i = row * a.N + sl.idx[v];
        xs[0] = D::scalar(a.x, i);
        ds[0] = D::scalar(a.dy, i);
      }
      float o[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xh = (xs[e] - mu) * r;
        const float g = ds[e] * gam[v][e];
        o[e] = r * fmaf(-xh, c1, g - c2);
        accg[v][e] = fmaf(ds[e], xh, accg[v][e]);
        if constexpr (LN) accb[v][e] += ds[e];
      }
      if (a.dres) {  // gradient arriving at a fused residual sum
        if constexpr (VEC) {
          const u32x4 gv = ld16_stream(a.dres, row * a.nvec + sl.idx[v]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) o[e] += D::get(gv, e);
        } else {
          o[0] += D::scalar(a.dres, row * a.N + sl.idx[v]);
        }
      }
      if constexpr (VEC) {
        st16_stream(a.dx, row * a.nvec + sl.idx[v], D::pack(o));
      } else {
        D::put_scalar(a.dx, row * a.N + sl.idx[v], o[0]);
      }
    }
  }

  float* const out_g = a.part_g + static_cast<int64_t>(blockIdx.y) * a.N;
  float* const out_b = a.part_b + static_cast<int64_t>(blockIdx.y) * a.N;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (!sl.own[v]) continue;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int64_t col = sl.idx[v] * EPV + e;
      out_g[col] = accg[v][e];
      if constexpr (LN) out_b[col] = accb[v][e];
    }
  }
}

}  // namespace

// --------------------------------------------------------------------- launchers
// (kind, type pair, vector or scalar) -> the kernel instance.
#define RN_SPLIT_DISPATCH(kind, tc, vec, CALL)                                          \
  do {                                                                                  \
    const bool ln_ = kind == 1;                                                         \
    if (vec) {                                                                          \
      if (tc == kTcF32) { if (ln_) CALL(true, F32, F32, true) else CALL(false, F32, F32, true) } \
      if (tc == kTcBF16) { if (ln_) CALL(true, BF16, BF16, true) else CALL(false, BF16, BF16, true) } \
      if (tc == kTcF16) { if (ln_) CALL(true, F16, F16, true) else CALL(false, F16, F16, true) } \
      if (tc == kTcBF16F32) { if (ln_) CALL(true, BF16, F32, true) else CALL(false, BF16, F32, true) } \
      if (tc == kTcF16F32) { if (ln_) CALL(true, F16, F32, true) else CALL(false, F16, F32, true) } \
    } else {                                                                            \
      if (tc == kTcF32) { if (ln_) CALL(true, F32, F32, false) else CALL(false, F32, F32, false) } \
      if (tc == kTcBF16) { if (ln_) CALL(true, BF16, BF16, false) else CALL(false, BF16, BF16, false) } \
      if (tc == kTcF16) { if (ln_) CALL(true, F16, F16, false) else CALL(false, F16, F16, false) } \
      if (tc == kTcBF16F32) { if (ln_) CALL(true, BF16, F32, false) else CALL(false, BF16, F32, false) } \
      if (tc == kTcF16F32) { if (ln_) CALL(true, F16, F32, false) else CALL(false, F16, F32, false) } \
    }                                                                                   \
  } while (0)

namespace {

MergeArgs merge_args(const float* rowp, float* out, int64_t M, int32_t N, int32_t slices,
                     int32_t slice_elems, float inv_n) {
  MergeArgs m;
  m.rowp = rowp;
  m.out = out;
  m.mean = nullptr;
  m.rstd = nullptr;
  m.M = M;
  m.N = N;
  m.slices = slices;
  m.slice_elems = slice_elems;
  m.inv_n = inv_n;
  m.eps = 0.0f;
  return m;
}

template <int MODE>
hipError_t launch_merge(const MergeArgs& m, int grid, hipStream_t s) {
  hipLaunchKernelGGL((rowmerge_kernel<MODE>), dim3(grid), dim3(kMergeBlock), 0, s, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_split(int kind, int tc, bool vec, const FwdArgs& a, int slices,
                            int row_blocks, int merge_grid, hipStream_t s) {
  const dim3 grid(slices, row_blocks);
  hipError_t e = hipErrorInvalidValue;
#define RN_CALL(LN, D, P, VEC)                                                                  \
  {                                                                                             \
    hipLaunchKernelGGL((fwd_slicestats_kernel<LN, D, P, VEC>), grid, dim3(kSliceBlock), 0, s, a); \
    e = hipGetLastError();                                                                      \
  }
  RN_SPLIT_DISPATCH(kind, tc, vec, RN_CALL);
#undef RN_CALL
  if (e != hipSuccess) return e;
  const int epu = vec ? (tc == kTcF32 ? 4 : 8) : 1;
  MergeArgs m = merge_args(a.rowp, a.rowtab, a.M, a.N, slices, slice_units(vec) * epu, a.inv_n);
  m.mean = a.mean;
  m.rstd = a.rstd;
  m.eps = a.eps;
  e = kind == 1 ? launch_merge<1>(m, merge_grid, s) : launch_merge<0>(m, merge_grid, s);
  if (e != hipSuccess) return e;
  e = hipErrorInvalidValue;
#define RN_CALL(LN, D, P, VEC)                                                                  \
  {                                                                                             \
    hipLaunchKernelGGL((fwd_slicenorm_kernel<LN, D, P, VEC>), grid, dim3(kSliceBlock), 0, s, a); \
    e = hipGetLastError();                                                                      \
  }
  RN_SPLIT_DISPATCH(kind, tc, vec, RN_CALL);
#undef RN_CALL
  return e;
}

hipError_t launch_bwd_split(int kind, int tc, bool vec, const BwdArgs& a, int slices,
                            int row_blocks, int64_t rows_per_block, int col_blocks,
                            int64_t col_rows, int merge_grid, hipStream_t s) {
  BwdArgs a1 = a;
  a1.rows_per_block = rows_per_block;
  BwdArgs a2 = a;
  a2.rows_per_block = col_rows;
  hipError_t e = hipErrorInvalidValue;
  dim3 grid(slices, row_blocks);
#define RN_CALL(LN, D, P, VEC)                                                                 \
  {                                                                                            \
    hipLaunchKernelGGL((bwd_slicedot_kernel<LN, D, P, VEC>), grid, dim3(kSliceBlock), 0, s, a1); \
    e = hipGetLastError();                                                                     \
  }
  RN_SPLIT_DISPATCH(kind, tc, vec, RN_CALL);
#undef RN_CALL
  if (e != hipSuccess) return e;
  const MergeArgs m = merge_args(a.rowp, a.rowc, a.M, a.N, slices, 0, a.inv_n);
  e = kind == 1 ? launch_merge<3>(m, merge_grid, s) : launch_merge<2>(m, merge_grid, s);
  if (e != hipSuccess) return e;
  e = hipErrorInvalidValue;
  grid = dim3(slices, col_blocks);
#define RN_CALL(LN, D, P, VEC)                                                              \
  {                                                                                         \
    hipLaunchKernelGGL((colslice_kernel<LN, D, P, VEC>), grid, dim3(kSliceBlock), 0, s, a2); \
    e = hipGetLastError();                                                                  \
  }
  RN_SPLIT_DISPATCH(kind, tc, vec, RN_CALL);
#undef RN_CALL
  return e;
}

}  // namespace rownorm
