// Split-row ("cluster") kernels for rows too long for one workgroup's registers.
//
// The pages note that very long rows cost Triton on H100 because it cannot reduce a
// row across cooperating SMs ("SOTA normalization performance with torch.compile",
// theaicatchup.com, "How Did Torch.compile Catch Quack?").  Here C workgroups share
// each row: workgroup k of a cluster owns the k-th column slice of every
// row the cluster handles, keeps its slice of gamma (and beta) in registers for all of
// them, and, in the backward, its slice's dgamma/dbeta column sums as well.  Per row, each
// member reduces its slice inside the workgroup (DPP + LDS), publishes the partial sums,
// waits for the other members' partials of the same row and combines all C of them in
// member order (identical, deterministic bits in every member).  HBM sees every element
// once, as in the register-resident kernels.
//
// Exchange: every step of rows has its own slots, one 64-bit word per member and value
// (at least two per member), each holding a 32-bit float beside one half of a 64-bit tag
// (the high half in even words, the low half in odd ones).  The tag derives from the
// call's tag base and the step.  A member writes its words with relaxed agent-scope
// atomic stores and readers spin on agent-scope atomic loads until all of a member's
// words carry the step's tag, so the words validate themselves (a reader that sees some
// of them before the others just polls again) and no ordering between words is needed.
// Each slot is written once per launch.  Every call outside graph capture has its own
// tag base (a hash of a per-process epoch that counts up from a random start), so words
// left by earlier calls, or any other contents of the workspace, match a step's tag with
// a probability of 2^-62 per read, and the slots are not cleared between calls.  Calls
// captured into a graph would replay one tag base, so for them a fill kernel captured
// with the call zeroes the slots first (a zero word never matches: each tag half has its
// top bit set).
//
// The kernels are launched like any other (a cooperative launch costs about 25 us of
// idle device time around every call on this platform), with a grid the device can hold
// at once, so the members of a cluster normally run together.  Nothing depends on it:
// a member that has polled another's words `spin_limit` times leaves the pipelined loop,
// finishes its steps one at a time (polling 256 times fewer per word) and computes any
// partial sums that do not arrive itself, from the same data with the same operations
// (floating-point contraction off), so the result has the same bits and every wait ends.
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

// Tag of a step's words: the call's 64-bit tag base (a hash of its epoch, made on the
// host) plus (step + 1) times an odd constant, with the top bit of each 32-bit half set
// so that a zero word never matches.  Two calls' tags for the same step differ unless
// their bases do; a word of another call and step matches only if the difference of the
// bases equals a multiple of the constant that the steps fix, a chance of 2^-62.
struct Tag {
  uint32_t hi, lo;
};
__device__ inline Tag step_tag(uint64_t base, int64_t step) {
  const uint64_t h = base + (static_cast<uint64_t>(step) + 1) * 0x9E3779B97F4A7C15ull;
  return Tag{static_cast<uint32_t>(h >> 32) | 0x80000000u, static_cast<uint32_t>(h) | 0x80000000u};
}

// Words a member writes per step for K values: one per value, at least two, so that the
// step's words together carry both halves of its tag.
template <int K>
constexpr int kWords = K < 2 ? 2 : K;

// Word j of a member's step: [tag half | value], the high half of the tag in even words
// and the low half in odd ones; with one value, the second word repeats it.
template <int K>
__device__ inline unsigned long long step_word(Tag tag, int j, const float (&v)[K]) {
  const uint32_t half = (j & 1) ? tag.lo : tag.hi;
  return (static_cast<unsigned long long>(half) << 32) | __float_as_uint(v[j < K ? j : 0]);
}

// Whether a member's words of a step carry the step's tag (and, with one value, agree).
template <int K>
__device__ inline bool words_match(const unsigned long long (&w)[kWords<K>], Tag tag) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < kWords<K>; ++j)
    ok = ok && static_cast<uint32_t>(w[j] >> 32) == ((j & 1) ? tag.lo : tag.hi);
  if constexpr (K == 1) ok = ok && static_cast<uint32_t>(w[0]) == static_cast<uint32_t>(w[1]);
  return ok;
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
// all R rows of a step.  Every step has its own exchange slots: [member][kWords<K>]
// 64-bit words.
template <int K>
__device__ inline void publish_step(const ClusterArgs& c, int member, int step,
                                    const float (&mine)[K]) {
  if (threadIdx.x == 0) {
    constexpr int W = kWords<K>;
    unsigned long long* base = c.xchg + static_cast<int64_t>(step) * c.C * W + member * W;
    const Tag tag = step_tag(c.tag_base, step);
#pragma unroll
    for (int j = 0; j < W; ++j)
      __hip_atomic_store(base + j, step_word<K>(tag, j, mine), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Word j of member m's slots for `step`: a uniform base for the step plus a 32-bit offset
// that is opaque to the optimiser, so that no 64-bit per-lane address is kept live (and
// spilled) across the step loop, and the address is formed only where it is used.
template <int K>
__device__ inline unsigned long long* slot_ptr(const ClusterArgs& c, int step, uint32_t m, int j) {
  constexpr int W = kWords<K>;
  uint32_t ofs = (m * W + j) * 8u;
  asm volatile("" : "+v"(ofs));
  char* base = reinterpret_cast<char*>(c.xchg + static_cast<int64_t>(step) * c.C * W);
  return reinterpret_cast<unsigned long long*>(base + ofs);
}

template <int K>
__device__ inline void load_words(const ClusterArgs& c, int step, unsigned long long (&w)[kWords<K>]) {
#pragma unroll
  for (int j = 0; j < kWords<K>; ++j)
    w[j] = __hip_atomic_load(slot_ptr<K>(c, step, threadIdx.x, j), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Thread m < C reads member m's words of `step` ahead of the gather, so the round trip of
// the first poll overlaps other work instead of stalling the whole workgroup.
template <int K>
__device__ inline void prefetch_step(const ClusterArgs& c, int step,
                                     unsigned long long (&pre)[kWords<K>]) {
  if (threadIdx.x < c.C) load_words<K>(c, step, pre);
}

// Every member's K partials of `step` into xin[member * K + j] (thread m < C handles member
// m).  Prefetched words that already carry the step's tag are used as they are; otherwise
// the thread polls, at most `limit` times, until all of the member's words do (a reader
// that sees some of them before the others just polls again).  xok[m] records whether
// member m's words arrived.  The results are visible to the workgroup after its next
// barrier.
template <int K>
__device__ inline void resolve_step(const ClusterArgs& c, int step,
                                    const unsigned long long (&pre)[kWords<K>], float* xin,
                                    int* xok, uint32_t limit) {
  if (threadIdx.x < c.C) {
    const Tag tag = step_tag(c.tag_base, step);
    unsigned long long w[kWords<K>];
#pragma unroll
    for (int j = 0; j < kWords<K>; ++j) w[j] = pre[j];
    bool ok = limit != 0 && words_match<K>(w, tag);
    for (uint32_t n = 0; limit != 0 && !ok && n < limit; ++n) {
      __builtin_amdgcn_s_sleep(2);
      load_words<K>(c, step, w);
      ok = words_match<K>(w, tag);
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
      xin[threadIdx.x * K + j] = ok ? __uint_as_float(static_cast<uint32_t>(w[j])) : 0.0f;
    xok[threadIdx.x] = ok ? 1 : 0;
  }
}

// The members whose words did not arrive (a bit per member, the same in every thread),
// read after the barrier that follows resolve_step: the caller computes those partials
// itself.
__device__ inline unsigned missing_members(const ClusterArgs& c, const int* xok) {
  unsigned miss = 0;
  for (int m = 0; m < c.C; ++m) miss |= xok[m] ? 0u : (1u << m);
  return miss;
}

// resolve_step and missing_members with a barrier of their own.  The caller alternates
// between two xin / xok buffers, so values are never overwritten before every thread has
// read them.
template <int K>
__device__ inline unsigned gather_step(const ClusterArgs& c, int step,
                                       const unsigned long long (&pre)[kWords<K>], float* xin,
                                       int* xok, uint32_t limit) {
  resolve_step<K>(c, step, pre, xin, xok, limit);
  __syncthreads();
  return missing_members(c, xok);
}

// ------------------------------------------------------------------ partial row sums
// A member whose partners' words do not arrive computes their partial sums itself
// (fwd_missing / bwd_missing).  Both it and the partner perform the same operations in the
// same order with floating-point contraction off, so the result has the same bits either
// way.  The missing-partner paths are cold: their vector loops stay rolled (one vector
// live at a time) so that they take next to no registers from the pipelined step loop.

// Forward partial sums of a step's R rows over one slice, from an accessor X(i, v) of
// its vectors: RMSNorm sums of squares; LayerNorm slice sums and sums of squared
// deviations about the slice mean.  Reduced over the workgroup (identical in every thread).
template <bool LN, typename D, int T, int VPL, int R, typename XF>
__device__ __forceinline__ void fwd_partial(XF&& X, int slice_vecs, float slice_n,
                                            float (&out)[(LN ? 2 : 1) * R], float* red,
                                            int& parity) {
#pragma clang fp contract(off)
  constexpr int EPV = D::kPerVec;
  constexpr int NW = T / 64;
  constexpr int K = (LN ? 2 : 1) * R;
  if constexpr (LN) {
    float s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      s[i] = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) s[i] = D::sum(X(i, v), s[i]);
    }
    block_sum_n<NW, R>(s, red, parity);
    float m2[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float m_k = s[i] / slice_n;
      m2[i] = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const u32x4 xv = X(i, v);
        const bool mine = v * T + static_cast<int>(threadIdx.x) < slice_vecs;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float d = mine ? D::get_fresh(xv, e) - m_k : 0.0f;
          m2[i] = fmaf(d, d, m2[i]);
        }
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
      for (int v = 0; v < VPL; ++v) out[i] = D::sumsq(X(i, v), out[i]);
    }
    block_sum_n<NW, K>(out, red, parity);
  }
}

// The forward partials of the members in `miss` (a bit per member) for step st, computed
// from their slices (with ADD, the rounded residual sum those members write out), into
// xs[member * K + j]: fwd_partial's operations in its order.  Returns the updated
// reduction-buffer parity.
template <bool LN, typename D, int T, int VPL, int R, bool ADD>
__device__ __forceinline__ int fwd_missing(const FwdArgs& a, const ClusterArgs& c, unsigned miss,
                                           int st, float slice_n, float* red, float* xs,
                                           int parity) {
#pragma clang fp contract(off)
  constexpr int EPV = D::kPerVec;
  constexpr int NW = T / 64;
  constexpr int K = (LN ? 2 : 1) * R;
  const int tid = threadIdx.x;
  for (int m = 0; m < c.C; ++m) {
    if (!((miss >> m) & 1u)) continue;
    const int64_t mofs = static_cast<int64_t>(m) * c.slice_vecs;
    auto vec = [&](int i, int v) -> u32x4 {
      const int64_t row = static_cast<int64_t>(st) * R + i;
      const bool ok = v * T + tid < c.slice_vecs && row < a.M;
      const int64_t idx = row * a.nvec + mofs + v * T + tid;
      u32x4 xv = ok ? ld16_stream(a.x, idx) : zero16();
      if constexpr (ADD) xv = D::add(xv, ok ? ld16_stream(a.res, idx) : zero16());
      return xv;
    };
    float t[K];
    if constexpr (LN) {
      float sm[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        sm[i] = 0.0f;
#pragma unroll 1
        for (int v = 0; v < VPL; ++v) sm[i] = D::sum(vec(i, v), sm[i]);
      }
      block_sum_n<NW, R>(sm, red, parity);
      float m2[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float m_k = sm[i] / slice_n;
        m2[i] = 0.0f;
#pragma unroll 1
        for (int v = 0; v < VPL; ++v) {
          const u32x4 xv = vec(i, v);
          const bool mine = v * T + tid < c.slice_vecs;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float d = mine ? D::get_fresh(xv, e) - m_k : 0.0f;
            m2[i] = fmaf(d, d, m2[i]);
          }
        }
      }
      block_sum_n<NW, R>(m2, red, parity);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        t[2 * i] = sm[i];
        t[2 * i + 1] = m2[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        t[i] = 0.0f;
#pragma unroll 1
        for (int v = 0; v < VPL; ++v) t[i] = D::sumsq(vec(i, v), t[i]);
      }
      block_sum_n<NW, K>(t, red, parity);
    }
    if (tid == 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) xs[m * K + j] = t[j];
    }
  }
  __syncthreads();
  return parity;
}

// Backward row-sum terms of one 16-byte vector of a slice: s1 += g * xhat, s2 += g
// (g = dy * gamma; gfv, when given, is gamma unpacked), and the unpacked xhat and dy.
template <bool LN, bool kDot, typename D, typename PV>
__device__ __forceinline__ void bwd_vec_sums(const u32x4& xv, const u32x4& dv, const PV& gv,
                                             const float* gfv, float r, float mu, float& s1,
                                             float& s2, float (&xs)[D::kPerVec],
                                             float (&ds)[D::kPerVec]) {
#pragma clang fp contract(off)
  if constexpr (LN && kDot) s2 = D::dot(dv, gv.v, s2);
#pragma unroll
  for (int e = 0; e < D::kPerVec; ++e) {
    const float xh = (D::get_fresh(xv, e) - mu) * r;
    const float d = D::get_fresh(dv, e);
    const float gg = d * (gfv ? gfv[e] : gv.get_fresh(e));
    s1 = fmaf(gg, xh, s1);
    if constexpr (LN && !kDot) s2 += gg;
    xs[e] = xh;
    ds[e] = d;
  }
}

// The backward partial row sums of the members in `miss` for step st, computed from their
// slices of x, dy and gamma (no column sums: those are each member's own), into
// xs[member * K + j].  Returns the updated reduction-buffer parity.
template <bool LN, typename D, typename P, int T, int VPL, int R>
__device__ __forceinline__ int bwd_missing(const BwdArgs& a, const ClusterArgs& c, unsigned miss,
                                        int st, float* red, float* xs, int parity) {
  using PV = Param<D, P>;
  constexpr int EPV = D::kPerVec;
  constexpr int NW = T / 64;
  constexpr int K = 2 * R;
  constexpr bool kDot = !std::is_same<D, F32>::value && PV::kPacked;
  const int tid = threadIdx.x;
  for (int m = 0; m < c.C; ++m) {
    if (!((miss >> m) & 1u)) continue;
    const int64_t mofs = static_cast<int64_t>(m) * c.slice_vecs;
    float out[K];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t row = static_cast<int64_t>(st) * R + i;
      const float r = row < a.M ? a.rstd[row] : 0.0f;
      const float mu = (LN && row < a.M) ? a.mean[row] : 0.0f;
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll 1
      for (int v = 0; v < VPL; ++v) {
        const bool mine = v * T + tid < c.slice_vecs;
        const bool ok = mine && row < a.M;
        const int64_t idx = row * a.nvec + mofs + v * T + tid;
        const u32x4 xv = ok ? ld16_stream(a.x, idx) : zero16();
        const u32x4 dv = ok ? ld16_stream(a.dy, idx) : zero16();
        PV gv;
        if (mine) {
          gv.load(a.gamma, mofs + v * T + tid);
        } else {
          gv.clear();
        }
        float xs_[EPV], ds_[EPV];
        bwd_vec_sums<LN, kDot, D>(xv, dv, gv, nullptr, r, mu, s1, s2, xs_, ds_);
      }
      out[2 * i] = s1;
      out[2 * i + 1] = s2;
    }
    block_sum_n<NW, K>(out, red, parity);
    if (tid == 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) xs[m * K + j] = out[j];
    }
  }
  __syncthreads();
  return parity;
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
  // steps and step indices are 32-bit (the planner keeps M below 2^31)
  const int nsteps = static_cast<int>((a.M + R - 1) / R);

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
  __shared__ int xok[2][kMaxCluster];
  int parity = 0, xp = 0;

  // A step's x slices (with ADD, and the residual's): every access goes through a buffer
  // resource of the row's slice (rows past M get an empty one), so the loads are
  // unconditional and read zero where there is no data, and stores there are dropped.
  struct Stage {
    u32x4 x[R][VPL];
    u32x4 r[ADD ? R : 1][VPL];
  };
  const uint32_t slice_bytes = static_cast<uint32_t>(c.slice_vecs) * 16u;
  const int M32 = static_cast<int>(a.M);
  auto slice = [&](const void* base, int row) {
    return make_rsrc(static_cast<const char*>(base) + (static_cast<int64_t>(row) * a.nvec + vofs) * 16,
                     row < M32 ? slice_bytes : 0u);
  };
  const uint32_t lane_ofs = static_cast<uint32_t>(tid) * 16u;
  auto load = [&](int st, Stage& sb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = st * R + i;
      const rsrc_t rx = slice(a.x, row);
#pragma unroll
      for (int v = 0; v < VPL; ++v) sb.x[i][v] = buf_ld16(rx, lane_ofs + v * T * 16);
      if constexpr (ADD) {
        const rsrc_t rr = slice(a.res, row);
#pragma unroll
        for (int v = 0; v < VPL; ++v) sb.r[i][v] = buf_ld16(rr, lane_ofs + v * T * 16);
      }
    }
  };
  // With ADD the row normalized is the rounded sum x + res, which is also written out.
  auto form_sum = [&](int st, Stage& sb) {
    if constexpr (ADD) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const rsrc_t rs = slice(a.sum, st * R + i);
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          sb.x[i][v] = D::add(sb.x[i][v], sb.r[i][v]);
          buf_st16(rs, lane_ofs + v * T * 16, sb.x[i][v]);
        }
      }
    }
  };
  // This member's partial sums of a step's rows (fwd_partial, reduced over the workgroup).
  auto partial = [&](const Stage& sb, float (&out)[K]) {
    fwd_partial<LN, D, T, VPL, R>([&](int i, int v) -> u32x4 { return sb.x[i][v]; },
                                  c.slice_vecs, slice_n, out, red, parity);
  };
  // y of a step's rows from the gathered partials of every member (contraction off: the
  // statistics come out the same wherever this runs).
  auto emit_y = [&](const Stage& sb, int st, const float* xs) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = st * R + i;
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
      if (member == 0 && tid == 0 && row < M32) {
        if (a.rstd) a.rstd[row] = r;
        if constexpr (LN) {
          if (a.mean) a.mean[row] = mu;
        }
      }
      const rsrc_t ry = slice(a.y, row);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float f = D::get_fresh(sb.x[i][v], e);
          if constexpr (LN) {
            o[e] = fmaf((f - mu) * r, g[v].get_fresh(e), b[v].get_fresh(e));
          } else {
            o[e] = f * r * g[v].get_fresh(e);
          }
        }
        buf_st16(ry, lane_ofs + v * T * 16, D::pack(o));
      }
    }
  };

  // Three steps live in registers: b[k0] waits for the exchange, b[k1] is reduced and
  // published this iteration and b[k2] is being loaded, so the exchange round trip of a
  // step overlaps a step of work.  The roles rotate through fixed registers (the loop body
  // is unrolled three times), so no step's data is copied while its loads are in flight.
  constexpr int S = 3;
  Stage sg[S];
  int st = cl;
  if (st >= nsteps) return;
  load(st, sg[0]);
  load(st + c.nclusters, sg[1]);
  {
    float mine[K];
    form_sum(st, sg[0]);
    partial(sg[0], mine);
    publish_step<K>(c, member, st, mine);
  }
  // Where step s2's loads are issued: before step s1's reduction (so they are in flight
  // during it), or after its publication (1024-lane members).
  constexpr bool kLoadFirst = T < 1024;
  // One pipelined step with compile-time stage roles; false when the loop is to end (no
  // steps left, or a partner is late: then st is the step to finish in the tail).
  auto pipe_step = [&](auto k0_) -> bool {
    constexpr int k0 = decltype(k0_)::value;
    constexpr int k1 = (k0 + 1) % S, k2 = (k0 + 2) % S;
    if (st >= nsteps) return false;
    const int s1 = st + c.nclusters, s2 = st + 2 * c.nclusters;
    unsigned long long pre[kWords<K>];
    prefetch_step<K>(c, st, pre);
    if constexpr (kLoadFirst) load(s2, sg[k2]);
    {
      float mine[K];
      form_sum(s1, sg[k1]);
      partial(sg[k1], mine);
      if (s1 < nsteps) publish_step<K>(c, member, s1, mine);
    }
    if constexpr (!kLoadFirst) load(s2, sg[k2]);
    float* xs = xin[xp];
    int* xk = xok[xp];
    xp ^= 1;
    if (gather_step<K>(c, st, pre, xs, xk, c.spin_limit)) return false;  // a partner is late
    emit_y(sg[k0], st, xs);
    st += c.nclusters;
    return true;
  };
  while (pipe_step(std::integral_constant<int, 0>{}) && pipe_step(std::integral_constant<int, 1>{}) &&
         pipe_step(std::integral_constant<int, 2>{})) {
  }
  // The rest of the steps, one at a time, computing any partial that does not arrive
  // (reached only when a partner's words are late).  Steps before `done` have had this
  // member's partials formed and published by the loop above; the residual sum of a step
  // is formed again (and written again, with the same values).
  if (st < nsteps) {
    const int done = st + 2 * c.nclusters;
    const uint32_t tail_limit = c.spin_limit >> 8;  // a late partner: wait less from now on
    for (; st < nsteps; st += c.nclusters) {
      Stage sb;
      load(st, sb);
      form_sum(st, sb);
      if (st >= done) {
        float mine[K];
        partial(sb, mine);
        publish_step<K>(c, member, st, mine);
      }
      unsigned long long pre[kWords<K>];
      prefetch_step<K>(c, st, pre);
      float* xs = xin[xp];
      int* xk = xok[xp];
      xp ^= 1;
      const unsigned miss = gather_step<K>(c, st, pre, xs, xk, tail_limit);
      if (miss) parity = fwd_missing<LN, D, T, VPL, R, ADD>(a, c, miss, st, slice_n, red, xs, parity);
      emit_y(sb, st, xs);
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
  // steps and step indices are 32-bit (the planner keeps M below 2^31)
  const int nsteps = static_cast<int>((a.M + R - 1) / R);

  // Per-column partial sums of the member's slice: registers, or (LACC, wide members)
  // LDS words private to each lane, [dgamma|dbeta][vector][4-column chunk][lane].
  constexpr bool LACC = bwd_lds_acc(LN, EPV, T, VPL);
  constexpr int CH = EPV / 4;
  constexpr int RV = LACC ? 1 : VPL;
  __shared__ float4 lacc[LACC ? (LN ? 2 : 1) * VPL * CH * T : 1];
  auto lidx = [&](int which, int v, int h) { return ((which * VPL + v) * CH + h) * T + tid; };

  bool own[VPL];
  // gamma kept in registers (the slice is the same for every row), also unpacked except
  // in 1024-lane members holding 16+ elements per lane, which have no registers for that
  constexpr bool GF = !(T == 1024 && VPL * EPV >= 16);
  PV g[VPL];
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
    if constexpr (GF) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) gf[v][e] = g[v].get(e);
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
  __shared__ int xok[2][kMaxCluster];
  int parity = 0, xp = 0;

  // A step's x and dy slices and its rows' saved statistics, loaded together.  Every
  // access goes through a buffer resource of the row's slice (rows past M get an empty
  // one), so the loads are unconditional and read zero where there is no data.
  struct Stage {
    u32x4 x[R][VPL], d[R][VPL];
    u32x4 g2[ADD ? R : 1][VPL];  // ADD: gradient arriving at the residual sum
    float r[R], mu[R];
  };
  const uint32_t slice_bytes = static_cast<uint32_t>(c.slice_vecs) * 16u;
  const int M32 = static_cast<int>(a.M);
  auto slice = [&](const void* base, int row) {
    return make_rsrc(static_cast<const char*>(base) + (static_cast<int64_t>(row) * a.nvec + vofs) * 16,
                     row < M32 ? slice_bytes : 0u);
  };
  const uint32_t lane_ofs = static_cast<uint32_t>(tid) * 16u;
  auto load = [&](int st, Stage& sb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = st * R + i;
      const rsrc_t rx = slice(a.x, row), rd = slice(a.dy, row);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        sb.x[i][v] = buf_ld16(rx, lane_ofs + v * T * 16);
        sb.d[i][v] = buf_ld16(rd, lane_ofs + v * T * 16);
      }
      if constexpr (ADD) {
        const rsrc_t rg = slice(a.dres, row);
#pragma unroll
        for (int v = 0; v < VPL; ++v) sb.g2[i][v] = buf_ld16(rg, lane_ofs + v * T * 16);
      }
      const uint32_t sn = row < M32 ? 4u : 0u;
      sb.r[i] = buf_ldf(make_rsrc(a.rstd + row, sn), 0);
      sb.mu[i] = LN ? buf_ldf(make_rsrc(a.mean + row, sn), 0) : 0.0f;
    }
  };
  // This thread's partial row sums of g*xhat and g over the member's slice, for each row
  // of the step, and the slice's column contributions to dgamma/dbeta (which need no row
  // sums); the caller reduces the row sums over the workgroup.  Rows past M have zero x
  // and dy, so they add nothing.
  auto partial_sums = [&](const Stage& sb, float (&out)[K]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float r = sb.r[i];
      const float mu = sb.mu[i];
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        float xs[EPV], ds[EPV];
        bwd_vec_sums<LN, kDot, D>(sb.x[i][v], sb.d[i][v], g[v], GF ? gf[GF ? v : 0] : nullptr, r,
                                  mu, s1, s2, xs, ds);
        if constexpr (!LACC) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            accg[v][e] = fmaf(ds[e], xs[e], accg[v][e]);
            if constexpr (LN) accb[v][e] += ds[e];
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
  };
  auto partial = [&](const Stage& sb, float (&out)[K]) {
    partial_sums(sb, out);
    block_sum_n<NW, K>(out, red, parity);
  };
  // S steps live in registers: b[k0] waits for the exchange, the next S-3 are published,
  // one is reduced and published this iteration and one is being loaded, so the exchange
  // round trip of a step overlaps S-2 steps of work.  The stage roles rotate through
  // fixed registers (the loop body is unrolled S times), so no step's data is copied
  // while its loads are still in flight.
  constexpr int S = (T <= 512 && VPL * R <= 2 && !ADD) ? 4 : 3;
  Stage b[S];
  int st = cl;
  if (st < nsteps) {
#pragma unroll
    for (int k = 0; k < S - 1; ++k) load(st + k * c.nclusters, b[k]);
#pragma unroll
    for (int k = 0; k < S - 2; ++k) {
      const int sk = st + k * c.nclusters;
      if (sk < nsteps) {
        float mine[K];
        partial(b[k], mine);
        publish_step<K>(c, member, sk, mine);
      }
    }
  }
  // dx of a step's rows from the gathered partials of every member (contraction off, as
  // for the partials).  Stores past the slice or past M are dropped by the range check.
  auto emit_dx = [&](const Stage& sb, int st, const float* xs) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = st * R + i;
      float t1 = 0.0f, t2 = 0.0f;
      for (int j = 0; j < c.C; ++j) {
        t1 += xs[j * K + 2 * i];
        t2 += xs[j * K + 2 * i + 1];
      }
      const float r = sb.r[i];
      const float mu = sb.mu[i];
      // dx = r * (g - c2 - xhat * c1) = g * r + (xhat * (-r * c1) + (-r * c2)).
      const float nrc1 = -r * (t1 * a.inv_n);
      const float nrc2 = LN ? -r * (t2 * a.inv_n) : 0.0f;
      const rsrc_t ro = slice(a.dx, row);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float xh = (D::get_fresh(sb.x[i][v], e) - mu) * r;
          const float gg =
              D::get_fresh(sb.d[i][v], e) * (GF ? gf[GF ? v : 0][e] : g[v].get_fresh(e));
          o[e] = fmaf(gg, r, fmaf(xh, nrc1, nrc2));
          if constexpr (ADD) o[e] += D::get_fresh(sb.g2[i][v], e);
        }
        buf_st16(ro, lane_ofs + v * T * 16, D::pack(o));
      }
    }
  };

  // One pipelined step with compile-time stage roles; false when the loop is to end
  // (no steps left, or a partner is late: then st is the step to finish in the tail).
  // Order: wave 0 reads step st's exchange words, then step sl's loads are issued, then
  // step sp is reduced (in waves other than 0 it waits only for its own loads, issued one
  // step earlier) and published, and only then does wave 0 wait for the other members'
  // words of step st: a late partner never delays this member's own publication.
  // Where step sl's loads are issued: before step sp's reduction (so they are in flight
  // during it), or after its publication (1024-lane members, which measure faster so).
  constexpr bool kLoadFirst = T < 1024;
  auto pipe_step = [&](auto k0_) -> bool {
    constexpr int k0 = decltype(k0_)::value;
    constexpr int kp = (k0 + S - 2) % S, kl = (k0 + S - 1) % S;
    if (st >= nsteps) return false;
    const int sp = st + (S - 2) * c.nclusters, sl = st + (S - 1) * c.nclusters;
    unsigned long long pre[kWords<K>];
    prefetch_step<K>(c, st, pre);
    if constexpr (kLoadFirst) load(sl, b[kl]);
    float mine[K];
    partial_sums(b[kp], mine);
    block_sum_n<NW, K>(mine, red, parity);
    if (sp < nsteps) publish_step<K>(c, member, sp, mine);
    if constexpr (!kLoadFirst) load(sl, b[kl]);
    float* xs = xin[xp];
    int* xk = xok[xp];
    xp ^= 1;
    if (gather_step<K>(c, st, pre, xs, xk, c.spin_limit)) return false;  // a partner is late
    emit_dx(b[k0], st, xs);
    st += c.nclusters;
    return true;
  };
  while (pipe_step(std::integral_constant<int, 0>{}) && pipe_step(std::integral_constant<int, 1>{}) &&
         (S < 3 || pipe_step(std::integral_constant<int, 2 % S>{})) &&
         (S < 4 || pipe_step(std::integral_constant<int, 3 % S>{}))) {
  }
  // The rest of the steps, one at a time, computing any partial that does not arrive
  // (reached only when a partner's words are late).  Steps before `done` have had this
  // member's partial (and column sums) formed and published by the loop above.
  if (st < nsteps) {
    const int done = st + (S - 1) * c.nclusters;
    const uint32_t tail_limit = c.spin_limit >> 8;  // a late partner: wait less from now on
    for (; st < nsteps; st += c.nclusters) {
      Stage sb;
      load(st, sb);
      if (st >= done) {
        float mine[K];
        partial(sb, mine);
        publish_step<K>(c, member, st, mine);
      }
      unsigned long long pre[kWords<K>];
      prefetch_step<K>(c, st, pre);
      float* xs = xin[xp];
      int* xk = xok[xp];
      xp ^= 1;
      const unsigned miss = gather_step<K>(c, st, pre, xs, xk, tail_limit);
      if (miss) parity = bwd_missing<LN, D, P, T, VPL, R>(a, c, miss, st, red, xs, parity);
      emit_dx(sb, st, xs);
    }
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
hipError_t launch_split(K kernel, int grid, int block, const A& a, const ClusterArgs& c,
                        hipStream_t s) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, a, c);
  return hipGetLastError();
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
    return a.res ? launch_split(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, grid, T_, a, \
                               c, s)                                                     \
                 : launch_split(fwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, grid, T_, a, \
                               c, s);
  RN_CLUSTER_FWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

hipError_t RN_BWD_LAUNCHER(int t, int vpl, int rows, const BwdArgs& a, const ClusterArgs& c, int grid,
                           hipStream_t s) {
#define RN_CASE(T_, V_, R_)                                                              \
  if (t == T_ && vpl == V_ && rows == R_)                                                \
    return a.dres ? launch_split(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, true>, grid, T_, a, \
                                c, s)                                                    \
                  : launch_split(bwd_cluster_kernel<kLN, DT, PT, T_, V_, R_, false>, grid, T_, a, \
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
