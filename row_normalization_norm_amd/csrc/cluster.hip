// Split-row ("cluster") kernels for rows too long for one workgroup's registers.
//
// The pages note that very long rows cost Triton on H100 because it cannot reduce a
// row across cooperating SMs ("SOTA normalization performance with torch.compile",
// theaicatchup.com, "How Did Torch.compile Catch Quack?").  Here C co-resident
// workgroups share each row: workgroup k of a cluster owns the k-th column slice of every
// row the cluster handles, keeps its slice of gamma (and beta) in registers for all of
// them, and, in the backward, its slice's dgamma/dbeta column sums as well.  Per row, each
// member reduces its slice inside the workgroup (DPP + LDS), publishes the partial sums,
// waits for the other members' partials of the same row and combines all C of them in
// member order (identical, deterministic bits in every member).  HBM sees every element
// once, as in the register-resident kernels.
//
// Exchange: every row has its own slots, one per member, of 64-bit words each holding a
// 32-bit tag (derived from the row index, never 0) and a 32-bit float.  A member writes
// its words with relaxed agent-scope atomic stores and readers spin on agent-scope
// atomic loads until the tag matches, so every word validates itself and no ordering
// between different words is needed.  The slots are zeroed by a fill kernel before each
// launch and each is written once per launch.
// Co-residency of all workgroups is guaranteed by a cooperative launch; every wait is
// bounded, and a timed-out wait yields NaN (and sets a status word) instead of hanging.
//
// LayerNorm statistics merge per-slice (sum, sum of squared deviations about the slice
// mean) with the pairwise-update formula of Chan, Golub and LeVeque, so the variance is
// exact for constant rows and free of mean(x^2) - mean^2 cancellation.
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

__device__ inline uint32_t row_tag(int64_t row) {
  return static_cast<uint32_t>((row + 1) & 0x7FFFFFFF) | 0x80000000u;
}

__device__ inline void publish(unsigned long long* slot, uint32_t tag, float v) {
  const unsigned long long w = (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
  __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until the slot carries `tag`.  Gives up after `limit` polls, or as soon as any
// wait of the launch has given up (the status word is sticky), so a failed exchange
// costs one time-out per launch, not one per row; the result is then NaN.
__device__ inline float wait_for(unsigned long long* slot, uint32_t tag, uint32_t limit,
                                 unsigned* status) {
  for (uint32_t n = 0;; ++n) {
    const unsigned long long w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<uint32_t>(w >> 32) == tag) return __uint_as_float(static_cast<uint32_t>(w));
    if (n >= limit) {
      atomicOr(status, 1u);
      return __builtin_nanf("");
    }
    if ((n & 63) == 63 &&
        __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return __builtin_nanf("");
    __builtin_amdgcn_s_sleep(2);
  }
}

// Sum of K values over the workgroup at once (one barrier), identical in every thread.
// red: 2 * NW * K floats, alternated by `parity`.
template <int NW, int K>
__device__ inline void block_sum_n(float (&v)[K], float* red, int& parity) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = group_sum<64>(v[k]);
  if constexpr (NW > 1) {
    float* buf = red + parity * NW * K;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) buf[(threadIdx.x >> 6) * K + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += buf[w * K + k];
      v[k] = t;
    }
    parity ^= 1;
  }
}

// A cluster works in steps of R consecutive rows: step t covers rows t*R .. t*R+R-1, and
// cluster cl takes steps cl, cl + nclusters, ...  One reduction and one exchange serve
// all R rows of a step.  Every step has its own exchange slots: [member][K] 64-bit words.
template <int K>
__device__ inline void publish_step(const ClusterArgs& c, int member, int64_t step,
                                    const float (&mine)[K]) {
  if (threadIdx.x == 0) {
    unsigned long long* base = c.xchg + step * c.C * K;
#pragma unroll
    for (int j = 0; j < K; ++j) publish(base + member * K + j, row_tag(step), mine[j]);
  }
}

// Thread m < C reads member m's K words of `step` ahead of the gather, so the round trip
// of the first poll overlaps other work instead of stalling the whole workgroup.
template <int K>
__device__ inline void prefetch_step(const ClusterArgs& c, int64_t step,
                                     unsigned long long (&pre)[K]) {
  if (threadIdx.x < c.C) {
    unsigned long long* base = c.xchg + step * c.C * K;
#pragma unroll
    for (int j = 0; j < K; ++j)
      pre[j] = __hip_atomic_load(base + threadIdx.x * K + j, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Gather every member's K partials of `step` into xin[member * K + j]; visible to the whole
// workgroup after the barrier.  A prefetched word that already carries the step's tag is
// used as is; otherwise the thread polls.  The caller alternates between two xin buffers,
// so values are never overwritten before every thread has read them.
template <int K>
__device__ inline void gather_step(const ClusterArgs& c, int64_t step,
                                   const unsigned long long (&pre)[K], float* xin) {
  if (threadIdx.x < c.C) {
    unsigned long long* base = c.xchg + step * c.C * K;
    const uint32_t tag = row_tag(step);
#pragma unroll
    for (int j = 0; j < K; ++j)
      xin[threadIdx.x * K + j] =
          static_cast<uint32_t>(pre[j] >> 32) == tag
              ? __uint_as_float(static_cast<uint32_t>(pre[j]))
              : wait_for(base + threadIdx.x * K + j, tag, c.spin_limit, c.status);
  }
  __syncthreads();
}

// Each workgroup keeps several steps in registers: the forward publishes step t+1's partial
// sums and issues step t+2's loads before it waits for the other members' partials of step
// t, so the exchange round trip overlaps a step of work instead of stalling every step; the
// backward runs up to two steps ahead when its registers allow.

// --------------------------------------------------------------------------- forward
template <bool LN, typename D, typename P, int T, int VPL, int R, bool ADD>
__global__ __launch_bounds__(T) void fwd_cluster_kernel(const FwdArgs a, const ClusterArgs c) {
  using PV = Param<D, P>;
  constexpr int EPV = D::kPerVec;
  constexpr int NW = T / 64;
  constexpr int K = (LN ? 2 : 1) * R;  // exchanged values per member and step
  const int tid = threadIdx.x;
  const int cl = blockIdx.x % c.nclusters;
  const int member = blockIdx.x / c.nclusters;
  const int64_t vofs = static_cast<int64_t>(member) * c.slice_vecs;
  const float slice_n = static_cast<float>(c.slice_vecs) * EPV;
  const int64_t nsteps = (a.M + R - 1) / R;

  bool own[VPL];
  PV g[VPL], b[LN ? VPL : 1];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    own[v] = v * T + tid < c.slice_vecs;
    if (own[v]) {
      g[v].load(a.gamma, vofs + v * T + tid);
      if constexpr (LN) b[v].load(a.beta, vofs + v * T + tid);
    } else {
      g[v].clear();
      if constexpr (LN) b[v].clear();
    }
  }

  __shared__ float red[2 * NW * R];
  __shared__ float xin[2][kMaxCluster * K];
  int parity = 0, xp = 0;

  // With ADD a step's residual slices come with x's and are added in before the step's
  // partial sums (the row normalized is the rounded sum, which is also written out).
  auto load = [&](int64_t st, u32x4 (&buf)[R][VPL], u32x4 (&rbuf)[ADD ? R : 1][VPL]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t row = st * R + i;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool ok = own[v] && row < a.M;
        const int64_t idx = row * a.nvec + vofs + v * T + tid;
        buf[i][v] = ok ? ld16_stream(a.x, idx) : zero16();
        if constexpr (ADD) rbuf[i][v] = ok ? ld16_stream(a.res, idx) : zero16();
      }
    }
  };
  auto form_sum = [&](int64_t st, u32x4 (&buf)[R][VPL], const u32x4 (&rbuf)[ADD ? R : 1][VPL]) {
    if constexpr (ADD) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t row = st * R + i;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          buf[i][v] = D::add(buf[i][v], rbuf[i][v]);
          if (own[v] && row < a.M) st16_stream(a.sum, row * a.nvec + vofs + v * T + tid, buf[i][v]);
        }
      }
    }
  };
  // This member's partial sums of a step's rows: RMSNorm sums of squares; LayerNorm slice
  // sums and sums of squared deviations about the slice means.
  auto partial = [&](const u32x4 (&buf)[R][VPL], float (&out)[K]) {
    if constexpr (LN) {
      float s[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        s[i] = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) s[i] = D::sum(buf[i][v], s[i]);
      }
      block_sum_n<NW, R>(s, red, parity);
      float m2[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float m_k = s[i] / slice_n;
        m2[i] = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float d = own[v] ? D::get_fresh(buf[i][v], e) - m_k : 0.0f;
            m2[i] = fmaf(d, d, m2[i]);
          }
      }
      block_sum_n<NW, R>(m2, red, parity);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        out[2 * i] = s[i];
        out[2 * i + 1] = m2[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        out[i] = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) out[i] = D::sumsq(buf[i][v], out[i]);
      }
      block_sum_n<NW, K>(out, red, parity);
    }
  };

  u32x4 b0[R][VPL], b1[R][VPL], b2[R][VPL];
  u32x4 r0[ADD ? R : 1][VPL], r1[ADD ? R : 1][VPL], r2[ADD ? R : 1][VPL];
  int64_t st = cl;
  if (st >= nsteps) return;
  load(st, b0, r0);
  if (st + c.nclusters < nsteps) load(st + c.nclusters, b1, r1);
  {
    float mine[K];
    form_sum(st, b0, r0);
    partial(b0, mine);
    publish_step<K>(c, member, st, mine);
  }
  for (; st < nsteps; st += c.nclusters) {
    const int64_t s1 = st + c.nclusters, s2 = st + 2 * c.nclusters;
    unsigned long long pre[K];
    prefetch_step<K>(c, st, pre);
    if (s1 < nsteps) {
      float mine[K];
      form_sum(s1, b1, r1);
      partial(b1, mine);
      publish_step<K>(c, member, s1, mine);
    }
    if (s2 < nsteps) load(s2, b2, r2);

    float* xs = xin[xp];
    xp ^= 1;
    gather_step<K>(c, st, pre, xs);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t row = st * R + i;
      if (row >= a.M) break;
      float mu = 0.0f, var;
      if constexpr (LN) {
        float tot = 0.0f;
        for (int j = 0; j < c.C; ++j) tot += xs[j * K + 2 * i];
        mu = tot * a.inv_n;
        float m2t = 0.0f;
        for (int j = 0; j < c.C; ++j) {
          const float dm = xs[j * K + 2 * i] / slice_n - mu;
          m2t += xs[j * K + 2 * i + 1] + slice_n * dm * dm;
        }
        var = m2t * a.inv_n;
      } else {
        float tot = 0.0f;
        for (int j = 0; j < c.C; ++j) tot += xs[j * K + i];
        var = tot * a.inv_n;
      }
      const float r = rsqrtf(var + a.eps);
      if (member == 0 && tid == 0) {
        if (a.rstd) a.rstd[row] = r;
        if constexpr (LN) {
          if (a.mean) a.mean[row] = mu;
        }
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (!own[v]) continue;
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float f = D::get_fresh(b0[i][v], e);
          if constexpr (LN) {
            o[e] = fmaf((f - mu) * r, g[v].get_fresh(e), b[v].get_fresh(e));
          } else {
            o[e] = f * r * g[v].get_fresh(e);
          }
        }
        st16_stream(a.y, row * a.nvec + vofs + v * T + tid, D::pack(o));
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        b0[i][v] = b1[i][v];
        b1[i][v] = b2[i][v];
        if constexpr (ADD) {
          r0[i][v] = r1[i][v];
          r1[i][v] = r2[i][v];
        }
      }
  }
}

// -------------------------------------------------------------------------- backward
template <bool LN, typename D, typename P, int T, int VPL, int R, bool ADD>
__global__ __launch_bounds__(T) void bwd_cluster_kernel(const BwdArgs a, const ClusterArgs c) {
  using PV = Param<D, P>;
  constexpr int EPV = D::kPerVec;
  constexpr int NW = T / 64;
  constexpr int K = 2 * R;  // exchanged values per member and step: (sum g*xhat, sum g) x R
  // Sums of dy * gamma straight from packed 16-bit words (dy and gamma of one type).
  constexpr bool kDot = !std::is_same<D, F32>::value && PV::kPacked;
  const int tid = threadIdx.x;
  const int cl = blockIdx.x % c.nclusters;
  const int member = blockIdx.x / c.nclusters;
  const int64_t vofs = static_cast<int64_t>(member) * c.slice_vecs;
  const int64_t nsteps = (a.M + R - 1) / R;

  // Per-column partial sums of the member's slice: registers, or (LACC, wide members)
  // LDS words private to each lane, [dgamma|dbeta][vector][4-column chunk][lane].
  constexpr bool LACC = bwd_lds_acc(LN, EPV, T, VPL);
  constexpr int CH = EPV / 4;
  constexpr int RV = LACC ? 1 : VPL;
  __shared__ float4 lacc[LACC ? (LN ? 2 : 1) * VPL * CH * T : 1];
  auto lidx = [&](int which, int v, int h) { return ((which * VPL + v) * CH + h) * T + tid; };

  bool own[VPL];
  PV g[VPL];
  // gamma unpacked once (the slice is the same for every row), except in 1024-lane
  // members holding 16+ elements per lane, which have no registers for it
  constexpr bool GF = !(T == 1024 && VPL * EPV >= 16);
  float gf[GF ? VPL : 1][EPV];
  float accg[RV][EPV], accb[LN ? RV : 1][EPV];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    own[v] = v * T + tid < c.slice_vecs;
    if (own[v]) {
      g[v].load(a.gamma, vofs + v * T + tid);
    } else {
      g[v].clear();
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if constexpr (GF) gf[v][e] = g[v].get(e);
    }
    if constexpr (LACC) {
#pragma unroll
      for (int w = 0; w < (LN ? 2 : 1); ++w)
#pragma unroll
        for (int h = 0; h < CH; ++h) lacc[lidx(w, v, h)] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        accg[v][e] = 0.0f;
        if constexpr (LN) accb[v][e] = 0.0f;
      }
    }
  }

  __shared__ float red[2 * NW * K];
  __shared__ float xin[2][kMaxCluster * K];
  int parity = 0, xp = 0;

  // A step's x and dy slices and its rows' saved statistics, loaded together.
  struct Stage {
    u32x4 x[R][VPL], d[R][VPL];
    u32x4 g2[ADD ? R : 1][VPL];  // ADD: gradient arriving at the residual sum
    float r[R], mu[R];
  };
  auto load = [&](int64_t st, Stage& sb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t row = st * R + i;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool ok = own[v] && row < a.M;
        const int64_t idx = row * a.nvec + vofs + v * T + tid;
        sb.x[i][v] = ok ? ld16_stream(a.x, idx) : zero16();
        sb.d[i][v] = ok ? ld16_stream(a.dy, idx) : zero16();
        if constexpr (ADD) sb.g2[i][v] = ok ? ld16_stream(a.dres, idx) : zero16();
      }
      sb.r[i] = row < a.M ? a.rstd[row] : 0.0f;
      sb.mu[i] = (LN && row < a.M) ? a.mean[row] : 0.0f;
    }
  };
  // Partial row sums of g*xhat and g over this member's slice, for each row of the step,
  // and the slice's column contributions to dgamma/dbeta (which need no row sums).
  // Rows past M have zero x and dy, so they add nothing.
  auto partial = [&](const Stage& sb, float (&out)[K]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float r = sb.r[i];
      const float mu = sb.mu[i];
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if constexpr (LN && kDot) s2 = D::dot(sb.d[i][v], g[v].v, s2);
        float xs[EPV], ds[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float xh = (D::get_fresh(sb.x[i][v], e) - mu) * r;
          const float d = D::get_fresh(sb.d[i][v], e);
          const float gg = d * (GF ? gf[GF ? v : 0][e] : g[v].get_fresh(e));
          s1 = fmaf(gg, xh, s1);
          if constexpr (LN && !kDot) s2 += gg;
          xs[e] = xh;
          ds[e] = d;
          if constexpr (!LACC) {
            accg[v][e] = fmaf(d, xh, accg[v][e]);
            if constexpr (LN) accb[v][e] += d;
          }
        }
        if constexpr (LACC) {
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            float4 t = lacc[lidx(0, v, h)];
            t.x = fmaf(ds[4 * h], xs[4 * h], t.x);
            t.y = fmaf(ds[4 * h + 1], xs[4 * h + 1], t.y);
            t.z = fmaf(ds[4 * h + 2], xs[4 * h + 2], t.z);
            t.w = fmaf(ds[4 * h + 3], xs[4 * h + 3], t.w);
            lacc[lidx(0, v, h)] = t;
            if constexpr (LN) {
              float4 u = lacc[lidx(1, v, h)];
              u.x += ds[4 * h];
              u.y += ds[4 * h + 1];
              u.z += ds[4 * h + 2];
              u.w += ds[4 * h + 3];
              lacc[lidx(1, v, h)] = u;
            }
          }
        }
      }
      out[2 * i] = s1;
      out[2 * i + 1] = s2;
    }
    block_sum_n<NW, K>(out, red, parity);
  };

  // S steps live in registers: b[0] waits for the exchange, b[1 .. S-3] are published,
  // b[S-2] is reduced and published this iteration and b[S-1] is being loaded, so the
  // exchange round trip of a step overlaps S-2 steps of work.
  constexpr int S = (T <= 512 && VPL * R <= 2 && !ADD) ? 4 : 3;
  Stage b[S];
  int64_t st = cl;
  if (st < nsteps) {
#pragma unroll
    for (int k = 0; k < S - 1; ++k) {
      const int64_t sk = st + k * c.nclusters;
      if (sk < nsteps) load(sk, b[k]);
    }
#pragma unroll
    for (int k = 0; k < S - 2; ++k) {
      const int64_t sk = st + k * c.nclusters;
      if (sk < nsteps) {
        float mine[K];
        partial(b[k], mine);
        publish_step<K>(c, member, sk, mine);
      }
    }
  }
  for (; st < nsteps; st += c.nclusters) {
    const int64_t sp = st + (S - 2) * c.nclusters, sl = st + (S - 1) * c.nclusters;
    unsigned long long pre[K];
    prefetch_step<K>(c, st, pre);
    if (sp < nsteps) {
      float mine[K];
      partial(b[S - 2], mine);
      publish_step<K>(c, member, sp, mine);
    }
    if (sl < nsteps) load(sl, b[S - 1]);

    float* xs = xin[xp];
    xp ^= 1;
    gather_step<K>(c, st, pre, xs);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t row = st * R + i;
      if (row >= a.M) break;
      float t1 = 0.0f, t2 = 0.0f;
      for (int j = 0; j < c.C; ++j) {
        t1 += xs[j * K + 2 * i];
        t2 += xs[j * K + 2 * i + 1];
      }
      const float r = b[0].r[i];
      const float mu = b[0].mu[i];
      // dx = r * (g - c2 - xhat * c1) = g * r + (xhat * (-r * c1) + (-r * c2)).
      const float nrc1 = -r * (t1 * a.inv_n);
      const float nrc2 = LN ? -r * (t2 * a.inv_n) : 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (!own[v]) continue;
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float xh = (D::get_fresh(b[0].x[i][v], e) - mu) * r;
          const float gg =
              D::get_fresh(b[0].d[i][v], e) * (GF ? gf[GF ? v : 0][e] : g[v].get_fresh(e));
          o[e] = fmaf(gg, r, fmaf(xh, nrc1, nrc2));
          if constexpr (ADD) o[e] += D::get_fresh(b[0].g2[i][v], e);
        }
        st16_stream(a.dx, row * a.nvec + vofs + v * T + tid, D::pack(o));
      }
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) b[k] = b[k + 1];
  }

  // This member's slice of the cluster's partial row.
  float* const out_g = a.part_g + static_cast<int64_t>(cl) * a.N;
  float* const out_b = LN ? a.part_b + static_cast<int64_t>(cl) * a.N : nullptr;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if (!own[v]) continue;
    const int64_t col0 = (vofs + v * T + tid) * EPV;
    if constexpr (LACC) {
      // each lane reads back only the LDS words it wrote
#pragma unroll
      for (int h = 0; h < CH; ++h) {
        *reinterpret_cast<float4*>(out_g + col0 + 4 * h) = lacc[lidx(0, v, h)];
        if constexpr (LN) *reinterpret_cast<float4*>(out_b + col0 + 4 * h) = lacc[lidx(1, v, h)];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        out_g[col0 + e] = accg[v][e];
        if constexpr (LN) out_b[col0 + e] = accb[v][e];
      }
    }
  }
}

template <typename K, typename A>
hipError_t launch_coop(K kernel, int grid, int block, const A& a, const ClusterArgs& c,
                       hipStream_t s) {
  A a_copy = a;
  ClusterArgs c_copy = c;
  void* args[] = {&a_copy, &c_copy};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block),
                                    args, 0, s);
}

template <typename K>
int occupancy(K kernel, int block) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel), block,
                                                   0) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

#define RN_CAT_(a, b, c, d) a##b##c##d
#define RN_CAT(a, b, c, d) RN_CAT_(a, b, c, d)
#define RN_FWD_LAUNCHER RN_CAT(launch_fwd_cluster_k, RN_KIND, _t, RN_TC)
#define RN_BWD_LAUNCHER RN_CAT(launch_bwd_cluster_k, RN_KIND, _t, RN_TC)
#define RN_FWD_OCC RN_CAT(occupancy_fwd_cluster_k, RN_KIND, _t, RN_TC)
#define RN_BWD_OCC RN_CAT(occupancy_bwd_cluster_k, RN_KIND, _t, RN_TC)

using DT = Types<RN_TC>::D;
using PT = Types<RN_TC>::P;
constexpr bool kLN = RN_KIND == 1;

hipError_t RN_FWD_LAUNCHER(int t, int vpl, int rows, const FwdArgs& a, const ClusterArgs& c, int grid,
                           hipStream_t s) {
#define RN_CASE(T_, V_, R_)                                                              \
  if (t == T_ && vpl == V_ && rows == R_)                                                \
    return a.res ? launch_coop(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, grid, T_, a, \
                               c, s)                                                     \
                 : launch_coop(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, grid, T_, a, \
                               c, s);
  RN_CLUSTER_FWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

hipError_t RN_BWD_LAUNCHER(int t, int vpl, int rows, const BwdArgs& a, const ClusterArgs& c, int grid,
                           hipStream_t s) {
#define RN_CASE(T_, V_, R_)                                                              \
  if (t == T_ && vpl == V_ && rows == R_)                                                \
    return a.dres ? launch_coop(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, grid, T_, a, \
                                c, s)                                                    \
                  : launch_coop(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, grid, T_, a, \
                                c, s);
  RN_CLUSTER_BWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

int RN_FWD_OCC(int t, int vpl, int rows, bool add) {
#define RN_CASE(T_, V_, R_)                                                         \
  if (t == T_ && vpl == V_ && rows == R_)                                           \
    return add ? occupancy(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, T_)   \
               : occupancy(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, T_);
  RN_CLUSTER_FWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return 0;
}

int RN_BWD_OCC(int t, int vpl, int rows, bool add) {
#define RN_CASE(T_, V_, R_)                                                         \
  if (t == T_ && vpl == V_ && rows == R_)                                           \
    return add ? occupancy(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, T_)   \
               : occupancy(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, T_);
  RN_CLUSTER_BWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return 0;
}

}  // namespace rownorm
