// Register-resident rows of any length and alignment (the GENERIC path for short rows:
// up to kGrowsFwdMaxElems elements forward, kGrowsBwdMaxElems backward).  Rows whose
// length or address does not allow 16-byte vectors are read with element loads, one row
// per 256-thread workgroup, element j of the row in lane j % 256 (consecutive lanes read
// consecutive elements, so every load and store instruction of a wavefront covers one
// contiguous span).  Each row is read from HBM once and kept in registers as fp32 across
// its reductions, as the vector kernels do; the next row's elements are loaded before the
// current one is reduced.
//
// The operations are those of the vector kernels (fwd_rows.hip, bwd_rows.hip): the forward
// of "Fused RMSNorm" (aryanashta.me, "What it is") and LayerNorm, and the backward with its
// two-stage dgamma/dbeta reduction (one partial row per workgroup, then colreduce_kernel).
//
// Built once per (kind, type pair) from RN_KIND / RN_TC on the command line.
#include <type_traits>

#include "launch.h"
#include "rownorm_dev.h"

#ifndef RN_KIND
#error "RN_KIND must be defined"
#endif
#ifndef RN_TC
#error "RN_TC must be defined"
#endif

namespace rownorm {
namespace {

constexpr int kGB = kGrowsBlock;
constexpr int kGW = kGrowsBlock / 64;  // wavefronts per workgroup (one row)

// Sum over the workgroup's row of one value per thread, identical in every thread.  buf
// holds kGW floats; callers alternate buffers so one barrier per reduction suffices.
__device__ inline float row_total(float v, float* buf) {
  v = group_sum<64>(v);
  if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kGW; ++w) t += buf[w];
  return t;
}

template <bool LN, typename D, typename P, int EPL>
__global__ __launch_bounds__(kGB) void fwd_grows_kernel(const FwdArgs a) {
  const int tid = threadIdx.x;
  const int N = a.N;
  // gamma/beta in registers (fp32)
  constexpr bool GREG = EPL <= 16;
  float gr[GREG ? EPL : 1], br[(GREG && LN) ? EPL : 1];
  if constexpr (GREG) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int j = k * kGB + tid;
      gr[k] = j < N ? P::scalar(a.gamma, j) : 0.0f;
      if constexpr (LN) br[k] = j < N ? P::scalar(a.beta, j) : 0.0f;
    }
  }
  // [which reduction][parity] buffers
  __shared__ float red[2 * 2 * kGW];
  int parity = 0;

  // Element j of a row: x, or with a fused residual add the sum x + res rounded to the
  // activation type.
  auto load = [&](int64_t row, float (&v)[EPL]) {
    const int64_t base = row * N;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int j = k * kGB + tid;
      if (row < a.M && j < N) {
        const float f = D::scalar(a.x, base + j);
        v[k] = a.res ? D::round(f + D::scalar(a.res, base + j)) : f;
      } else {
        v[k] = 0.0f;
      }
    }
  };
  float nv[EPL];
  if (blockIdx.x < a.M) load(blockIdx.x, nv);

  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t base = row * N;
    float v[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) v[k] = nv[k];
    if (row + gridDim.x < a.M) load(row + gridDim.x, nv);
    if (a.res) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        const int j = k * kGB + tid;
        if (j < N) D::put_scalar(a.sum, base + j, v[k]);
      }
    }
    // RMSNorm: mean of squares.  LayerNorm: the mean, then the mean squared deviation
    // from it, both from the registers.
    float mu = 0.0f, var;
    if constexpr (LN) {
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) s += v[k];
      mu = row_total(s, red + (0 * 2 + parity) * kGW) * a.inv_n;
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        const float d = k * kGB + tid < N ? v[k] - mu : 0.0f;
        ss = fmaf(d, d, ss);
      }
      var = row_total(ss, red + (1 * 2 + parity) * kGW) * a.inv_n;
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) ss = fmaf(v[k], v[k], ss);
      var = row_total(ss, red + (0 * 2 + parity) * kGW) * a.inv_n;
    }
    parity ^= 1;
    const float r = rsqrtf(var + a.eps);
    if (tid == 0) {
      if (a.rstd) a.rstd[row] = r;
      if constexpr (LN) {
        if (a.mean) a.mean[row] = mu;
      }
    }
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int j = k * kGB + tid;
      if (j < N) {
        const float gm = GREG ? gr[GREG ? k : 0] : P::scalar(a.gamma, j);
        float o;
        if constexpr (LN) {
          const float bt = GREG ? br[GREG ? k : 0] : P::scalar(a.beta, j);
          o = fmaf((v[k] - mu) * r, gm, bt);
        } else {
          o = v[k] * r * gm;
        }
        D::put_scalar(a.y, base + j, o);
      }
    }
  }
}

template <bool LN, typename D, typename P, int EPL>
__global__ __launch_bounds__(kGB) void bwd_grows_kernel(const BwdArgs a) {
  const int tid = threadIdx.x;
  const int N = a.N;
  const int mode = a.mode;
  float gr[EPL];
  float accg[EPL], accb[LN ? EPL : 1];
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const int j = k * kGB + tid;
    gr[k] = j < N ? P::scalar(a.gamma, j) : 0.0f;
    accg[k] = 0.0f;
    if constexpr (LN) accb[k] = 0.0f;
  }
  __shared__ float red[2 * 2 * kGW];
  int parity = 0;

  // A row's x, dy (and the gradient arriving at a fused residual sum), and its saved
  // statistics; rows past M and elements past N read as zero.
  auto load = [&](int64_t row, float (&xv)[EPL], float (&dv)[EPL], float (&rv)[EPL], float& rs,
                  float& mu) {
    const int64_t base = row * N;
    const bool rok = row < a.M;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int j = k * kGB + tid;
      const bool ok = rok && j < N;
      xv[k] = ok ? D::scalar(a.x, base + j) : 0.0f;
      dv[k] = ok ? D::scalar(a.dy, base + j) : 0.0f;
      rv[k] = (ok && a.dres) ? D::scalar(a.dres, base + j) : 0.0f;
    }
    rs = rok ? a.rstd[row] : 0.0f;
    mu = (LN && rok) ? a.mean[row] : 0.0f;
  };
  float nx[EPL], nd[EPL], nr[EPL], nrs = 0.0f, nmu = 0.0f;
  if (blockIdx.x < a.M) load(blockIdx.x, nx, nd, nr, nrs, nmu);

  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t base = row * N;
    float xv[EPL], dv[EPL], rv[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      xv[k] = nx[k];
      dv[k] = nd[k];
      rv[k] = nr[k];
    }
    const float r = nrs, mu = nmu;
    if (row + gridDim.x < a.M) load(row + gridDim.x, nx, nd, nr, nrs, nmu);

    // xhat = (x - mean) * rstd, g = dy * gamma; c1 = mean(g * xhat), c2 = mean(g).
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float xh = (xv[k] - mu) * r;
      const float g = dv[k] * gr[k];
      s1 = fmaf(g, xh, s1);
      if constexpr (LN) s2 += g;
    }
    s1 = row_total(s1, red + (0 * 2 + parity) * kGW);
    if constexpr (LN) s2 = row_total(s2, red + (1 * 2 + parity) * kGW);
    parity ^= 1;
    // dx = r * (g - c2 - xhat * c1) = g * r + (xhat * (-r * c1) + (-r * c2)).
    const float nrc1 = -r * (s1 * a.inv_n);
    const float nrc2 = LN ? -r * (s2 * a.inv_n) : 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int j = k * kGB + tid;
      if (j < N) {
        const float xh = (xv[k] - mu) * r;
        const float g = dv[k] * gr[k];
        float o = fmaf(g, r, fmaf(xh, nrc1, nrc2));
        if (a.dres) o += rv[k];
        D::put_scalar(a.dx, base + j, o);
        if (mode == kAtomicRow) {
          unsafeAtomicAdd(a.dgamma + j, dv[k] * xh);
          if constexpr (LN) unsafeAtomicAdd(a.dbeta + j, dv[k]);
        } else {
          accg[k] = fmaf(dv[k], xh, accg[k]);
          if constexpr (LN) accb[k] += dv[k];
        }
      }
    }
  }

  if (mode == kAtomicRow) return;
  // One partial row per workgroup (or, in the per-workgroup atomic mode, added into
  // dgamma/dbeta).
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const int j = k * kGB + tid;
    if (j < N) {
      if (mode == kTwoStage) {
        a.part_g[static_cast<int64_t>(blockIdx.x) * N + j] = accg[k];
        if constexpr (LN) a.part_b[static_cast<int64_t>(blockIdx.x) * N + j] = accb[k];
      } else {
        unsafeAtomicAdd(a.dgamma + j, accg[k]);
        if constexpr (LN) unsafeAtomicAdd(a.dbeta + j, accb[k]);
      }
    }
  }
}

}  // namespace

#define RN_CAT_(a, b, c, d) a##b##c##d
#define RN_CAT(a, b, c, d) RN_CAT_(a, b, c, d)
#define RN_FWD_LAUNCHER RN_CAT(launch_fwd_grows_k, RN_KIND, _t, RN_TC)
#define RN_BWD_LAUNCHER RN_CAT(launch_bwd_grows_k, RN_KIND, _t, RN_TC)

hipError_t RN_FWD_LAUNCHER(int epl, const FwdArgs& a, int grid, hipStream_t s) {
  constexpr bool kLN = RN_KIND == 1;
  using D = Types<RN_TC>::D;
  using P = Types<RN_TC>::P;
#define RN_CASE(E)                                                                        \
  if (epl == E) {                                                                         \
    hipLaunchKernelGGL((fwd_grows_kernel<kLN, D, P, E>), dim3(grid), dim3(kGB), 0, s, a); \
    return hipGetLastError();                                                             \
  }
  RN_GROWS_EPL(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

hipError_t RN_BWD_LAUNCHER(int epl, const BwdArgs& a, int grid, hipStream_t s) {
  constexpr bool kLN = RN_KIND == 1;
  using D = Types<RN_TC>::D;
  using P = Types<RN_TC>::P;
#define RN_CASE(E)                                                                        \
  if (epl == E) {                                                                         \
    hipLaunchKernelGGL((bwd_grows_kernel<kLN, D, P, E>), dim3(grid), dim3(kGB), 0, s, a); \
    return hipGetLastError();                                                             \
  }
  RN_GROWS_EPL(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

}  // namespace rownorm
