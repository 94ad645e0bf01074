// Forward kernel, register-resident rows (ROWS path).
//
// RMSNorm: rstd = 1/sqrt(mean(x^2) + eps), y = x * rstd * gamma ("Fused RMSNorm",
// aryanashta.me, "What it is").  LayerNorm: mean and biased variance of the row,
// y = (x - mean) * rstd * gamma + beta ("SOTA normalization performance with
// torch.compile", theaicatchup.com, "How Did Torch.compile Catch Quack?").
//
// One pass over HBM: the row is read once into registers with 16-byte loads, its sum
// and sum of squares are accumulated in fp32 (the "Fused RMSNorm" page, "How it works",
// on why low-precision accumulation drifts), reduced across the row's lanes (DPP inside
// a wavefront, LDS across wavefronts), then normalized from the registers and written
// once with 16-byte stores.
//
// Mapping: LPR lanes hold one row, VPL 16-byte vectors each.  Lane l of the row holds
// vectors v*LPR + l (v < VPL), so consecutive lanes touch consecutive 16 bytes and each
// wavefront-wide load instruction covers a contiguous 64*16-byte span of the row.
// LPR <= 64 packs 64/LPR rows into a wavefront (a row is one aligned lane group);
// LPR > 64 spreads a row over LPR/64 wavefronts.  The grid is persistent: workgroup b
// takes row groups b, b + gridDim.x, ...  gamma (and beta) are loaded once per
// workgroup and kept in registers when they fit.
//
// Built once per (kind, type pair): RN_KIND (0 RMSNorm, 1 LayerNorm) and RN_TC (the
// activation/parameter type pair, TypeCombo in launch.h) come from the compiler command
// line.
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

template <bool LN, typename D, typename P, int LPR, int VPL, bool ADD>
__global__ __launch_bounds__(fwd_block(LPR)) void fwd_rows_kernel(const FwdArgs a) {
  constexpr int BLOCK = fwd_block(LPR);
  constexpr int EPV = D::kPerVec;
  constexpr int ROWS = BLOCK / LPR;              // rows per workgroup per iteration
  constexpr int WPR = LPR > 64 ? LPR / 64 : 1;   // wavefronts per row
  using PV = Param<D, P>;
  // gamma/beta kept in registers when they take at most 32 VGPRs; fp32 parameters beside
  // 16-bit activations take twice that, which workgroups below 512 lanes can afford.
  constexpr int kParamRegs = (PV::kPacked ? 4 : 8) * VPL * (LN ? 2 : 1);
  constexpr bool GREG = kParamRegs <= 32 || (!PV::kPacked && LPR < 512 && kParamRegs <= 64);

  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int slot = tid / LPR;
  const int nvec = a.nvec;

  PV g[GREG ? VPL : 1];
  PV b[(GREG && LN) ? VPL : 1];
  if constexpr (GREG) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (vi < nvec) {
        g[v].load(a.gamma, vi);
        if constexpr (LN) b[v].load(a.beta, vi);
      } else {
        g[v].clear();
        if constexpr (LN) b[v].clear();
      }
    }
  }

  // Cross-wavefront partial sums.  Each reduction has its own pair of buffers, used by
  // alternate rows, so one barrier per reduction suffices: a wavefront cannot reuse a
  // buffer until every wavefront has passed the barrier of the following reduction,
  // i.e. has finished reading it.
  __shared__ float red[WPR > 1 ? 2 * 2 * ROWS * WPR : 1];
  int parity = 0;
  auto row_sum = [&](float v, int which) {
    constexpr int W = LPR < 64 ? LPR : 64;
    v = group_sum<W>(v);
    if constexpr (WPR > 1) {
      float* buf = red + ((which * 2 + parity) * ROWS + slot) * WPR;
      if ((tid & 63) == 0) buf[(tid >> 6) % WPR] = v;
      __syncthreads();
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) v += buf[w];
    }
    return v;
  };

  // The next row group's loads are issued before the current one is reduced, so HBM
  // reads stay in flight through the reduction and the stores.
  // With ADD the residual's vectors come with x's.
  auto load = [&](int64_t grp, u32x4 (&buf)[VPL], u32x4 (&rbuf)[ADD ? VPL : 1]) {
    const int64_t row = grp * ROWS + slot;
    if constexpr (VPL > 8) {
      // The widest mappings address the row from one opaque per-lane pointer.
      const u32x4* xp = opaque_ptr(static_cast<const u32x4*>(a.x) + (row * nvec + lane));
      const u32x4* rp =
          ADD ? opaque_ptr(static_cast<const u32x4*>(a.res) + (row * nvec + lane)) : nullptr;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool ok = row < a.M && v * LPR + lane < nvec;
        buf[v] = ok ? ld16_stream(xp, v * LPR) : zero16();
        if constexpr (ADD) rbuf[v] = ok ? ld16_stream(rp, v * LPR) : zero16();
      }
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int vi = v * LPR + lane;
        const bool ok = row < a.M && vi < nvec;
        buf[v] = ok ? ld16_stream(a.x, row * nvec + vi) : zero16();
        if constexpr (ADD) rbuf[v] = ok ? ld16_stream(a.res, row * nvec + vi) : zero16();
      }
    }
  };
  // Mappings with more than 8 vectors per lane (a whole 256 KiB row in one workgroup)
  // have no registers for a second row: each row is loaded at the top of its iteration,
  // and the other resident waves keep HBM busy meanwhile.
  constexpr bool PF = VPL <= 8;
  u32x4 nx[PF ? VPL : 1], nr[(PF && ADD) ? VPL : 1];
  if constexpr (PF) {
    if (blockIdx.x < a.groups) load(blockIdx.x, nx, nr);
  }

  for (int64_t grp = blockIdx.x; grp < a.groups; grp += gridDim.x) {
    const int64_t row = grp * ROWS + slot;
    const bool row_ok = row < a.M;
    const int64_t vbase = row * nvec;

    u32x4 xv[VPL], rv[ADD ? VPL : 1];
    if constexpr (PF) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        xv[v] = nx[v];
        if constexpr (ADD) rv[v] = nr[v];
      }
    } else {
      load(grp, xv, rv);
    }
    if constexpr (ADD) {
      // The row normalized is the residual sum, rounded to the activation type and
      // written out as it is formed.
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int vi = v * LPR + lane;
        xv[v] = D::add(xv[v], rv[v]);
        if (row_ok && vi < nvec) st16_stream(a.sum, vbase + vi, xv[v]);
      }
    }
    if constexpr (PF) {
      if (grp + gridDim.x < a.groups) load(grp + gridDim.x, nx, nr);
    }

    // RMSNorm: mean of squares.  LayerNorm: the mean, then the mean squared deviation
    // from it, both reduced from the registers (the row is read from memory once).
    // Deviations about the mean keep the variance exact for constant rows and free of
    // the cancellation of mean(x^2) - mean^2 when |mean| >> deviation.
    // Short rows keep the deviations from the mean for the output pass.
    constexpr bool KEEP = LN && VPL * EPV <= 32;
    float dev[KEEP ? VPL : 1][EPV];
    float mu = 0.0f, var;
    if constexpr (LN) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) s = D::sum(xv[v], s);
      mu = row_sum(s, 0) * a.inv_n;
      float ss = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool in_row = v * LPR + lane < nvec;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float d = in_row ? D::get(xv[v], e) - mu : 0.0f;
          ss = fmaf(d, d, ss);
          if constexpr (KEEP) dev[v][e] = d;
        }
      }
      var = row_sum(ss, 1) * a.inv_n;
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) ss = D::sumsq(xv[v], ss);
      var = row_sum(ss, 0) * a.inv_n;
    }
    if constexpr (WPR > 1) parity ^= 1;

    const float r = rsqrtf(var + a.eps);
    if (row_ok && lane == 0) {
      if (a.rstd) a.rstd[row] = r;
      if constexpr (LN) {
        if (a.mean) a.mean[row] = mu;
      }
    }

    // The widest mappings read gamma/beta per vector from opaque per-lane bases.
    constexpr int kPB = PV::kPacked ? 16 : 32;  // parameter bytes per 16-byte vector
    const char* gp = VPL > 8 ? opaque_ptr(static_cast<const char*>(a.gamma) + lane * kPB)
                             : static_cast<const char*>(a.gamma);
    const char* bp = (VPL > 8 && LN) ? opaque_ptr(static_cast<const char*>(a.beta) + lane * kPB)
                                     : static_cast<const char*>(a.beta);
    constexpr int kGS = VPL > 8 ? 0 : 1;  // lane term of the vector index for the plain bases
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (row_ok && vi < nvec) {
        PV gv, bv;
        if constexpr (GREG) {
          gv = g[v];
          if constexpr (LN) bv = b[v];
        } else {
          gv.load(gp, v * LPR + kGS * lane);
          if constexpr (LN) bv.load(bp, v * LPR + kGS * lane);
        }
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          // Unpack the packed row afresh (or reuse the kept deviations), so that only
          // the packed words stay live across the reductions.
          if constexpr (LN) {
            const float d = KEEP ? dev[KEEP ? v : 0][e] : D::get_fresh(xv[v], e) - mu;
            o[e] = fmaf(d * r, gv.get_fresh(e), bv.get_fresh(e));
          } else {
            o[e] = D::get_fresh(xv[v], e) * r * gv.get_fresh(e);
          }
        }
        st16_stream(a.y, vbase + vi, D::pack(o));
      }
    }
  }
}

// Pipelined forward for persistent grids (several row groups per workgroup) and mappings
// of up to 8 vectors per lane.  Every access to x, y, the residual, the saved
// statistics and gamma/beta is a raw buffer access through a resource of the row group
// (ROWS consecutive rows; groups past the last row get an empty one) or of the parameter
// vector, so no access sits under a branch: rows past M and the padding lanes of the last
// vector slot read zeros and drop their stores by the hardware's range check.  The row
// loop is unrolled twice with two fixed sets of registers, the next group's loads issued
// into one while the other is reduced and stored, so no register copy of an in-flight
// load is needed.  Both let the compiler count the memory operations still in flight and
// wait only for the loads a step uses: the stores of one group and the loads of the next
// stay in flight across the loop's back edge (a wait under a branch, or a copy of a
// register whose load is in flight, made it wait for all of them every iteration).
template <bool LN, typename D, typename P, int LPR, int VPL, bool ADD, int S>
__global__ __launch_bounds__(fwd_block(LPR)) void fwd_pipe_kernel(const FwdArgs a) {
  static_assert(VPL <= 8 && S >= 2, "pipelined mappings: up to 8 vectors per lane, 2+ stages");
  constexpr int BLOCK = fwd_block(LPR);
  constexpr int EPV = D::kPerVec;
  constexpr int ROWS = BLOCK / LPR;              // rows per row group
  constexpr int WPR = LPR > 64 ? LPR / 64 : 1;   // wavefronts per row
  using PV = Param<D, P>;
  // gamma/beta kept in registers when they take at most 32 VGPRs; fp32 parameters beside
  // 16-bit activations take twice that, which workgroups below 512 lanes can afford.
  constexpr int kParamRegs = (PV::kPacked ? 4 : 8) * VPL * (LN ? 2 : 1);
  constexpr bool GREG = kParamRegs <= 32 || (!PV::kPacked && LPR < 512 && kParamRegs <= 64);

  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int slot = tid / LPR;
  const int nvec = a.nvec;
  const uint32_t row_bytes = static_cast<uint32_t>(nvec) * 16u;

  // Byte offset of this lane's vector slot v inside its row group (and, without the row
  // term, inside the parameter vector).  Only the last slot can hold padding lanes (the
  // planner keeps the padding below one slot), which get an out-of-range offset.
  const bool last_in_row = (VPL - 1) * LPR + lane < nvec;
  const uint32_t row_ofs = static_cast<uint32_t>(slot) * row_bytes;
  auto col_ofs = [&](int v) -> uint32_t {
    const uint32_t o = static_cast<uint32_t>(v * LPR + lane) * 16u;
    return (v == VPL - 1 && !last_in_row) ? kOutOfRange : o;
  };
  auto ofs = [&](int v) -> uint32_t {
    return (v == VPL - 1 && !last_in_row) ? kOutOfRange
                                          : row_ofs + static_cast<uint32_t>(v * LPR + lane) * 16u;
  };
  // This workgroup's row groups: grp0, grp0 + G, ... below gend.  With a.persistent set,
  // the persistent workgroups stop at a.static_end and the rest take one group each
  // from there: the hardware starts those on the first CUs to finish, which evens out
  // the end of the kernel (workgroups start several microseconds apart).
  int64_t grp0, G, gend;
  if (a.persistent == 0) {
    grp0 = blockIdx.x;
    G = gridDim.x;
    gend = a.groups;
  } else if (static_cast<int>(blockIdx.x) < a.persistent) {
    grp0 = blockIdx.x;
    G = a.persistent;
    gend = a.static_end;
  } else {
    grp0 = a.static_end + (blockIdx.x - a.persistent);
    G = a.groups;
    gend = grp0 + 1;
  }
  // Resource over row group grp of a [M, N] tensor, and over its rows' statistics; empty
  // past this workgroup's groups.
  const int64_t end_rows = gend * ROWS < a.M ? gend * ROWS : a.M;
  auto group_rows = [&](int64_t grp) -> uint32_t {
    const int64_t left = end_rows - grp * ROWS;
    return left <= 0 ? 0u : left >= ROWS ? uint32_t(ROWS) : static_cast<uint32_t>(left);
  };
  auto group = [&](const void* base, int64_t grp) {
    return make_rsrc(static_cast<const char*>(base) + grp * ROWS * static_cast<int64_t>(row_bytes),
                     group_rows(grp) * row_bytes);
  };
  auto group_stat = [&](const float* base, int64_t grp) {
    return make_rsrc(base + grp * ROWS, base ? group_rows(grp) * 4u : 0u);
  };
  const uint32_t stat_ofs = lane == 0 ? static_cast<uint32_t>(slot) * 4u : kOutOfRange;

  constexpr int kPB = PV::kPacked ? 16 : 32;  // parameter bytes per activation vector
  const rsrc_t rg = make_rsrc(a.gamma, static_cast<uint32_t>(nvec) * kPB);
  const rsrc_t rb = make_rsrc(LN ? a.beta : a.gamma, static_cast<uint32_t>(nvec) * kPB);
  PV g[GREG ? VPL : 1];
  PV b[(GREG && LN) ? VPL : 1];
  if constexpr (GREG) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      g[v].load_buf(rg, col_ofs(v));
      if constexpr (LN) b[v].load_buf(rb, col_ofs(v));
    }
  }

  // Cross-wavefront partial sums.  Each reduction has its own pair of buffers, used by
  // alternate rows, so one barrier per reduction suffices: a wavefront cannot reuse a
  // buffer until every wavefront has passed the barrier of the following reduction,
  // i.e. has finished reading it.
  __shared__ float red[WPR > 1 ? 2 * 2 * ROWS * WPR : 1];
  int parity = 0;
  auto row_sum = [&](float v, int which) {
    constexpr int W = LPR < 64 ? LPR : 64;
    v = group_sum<W>(v);
    if constexpr (WPR > 1) {
      float* buf = red + ((which * 2 + parity) * ROWS + slot) * WPR;
      if ((tid & 63) == 0) buf[(tid >> 6) % WPR] = v;
      __syncthreads();
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) v += buf[w];
    }
    return v;
  };

  struct Stage {
    u32x4 x[VPL];
    u32x4 r[ADD ? VPL : 1];
  };
  auto load = [&](int64_t grp, Stage& st) {
    const rsrc_t rx = group(a.x, grp);
#pragma unroll
    for (int v = 0; v < VPL; ++v) st.x[v] = buf_ld16(rx, ofs(v));
    if constexpr (ADD) {
      const rsrc_t rr = group(a.res, grp);
#pragma unroll
      for (int v = 0; v < VPL; ++v) st.r[v] = buf_ld16(rr, ofs(v));
    }
  };

  auto process = [&](int64_t grp, Stage& st) {
    if constexpr (ADD) {
      // The row normalized is the residual sum, rounded to the activation type and
      // written out as it is formed.
      const rsrc_t rs = group(a.sum, grp);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        st.x[v] = D::add(st.x[v], st.r[v]);
        buf_st16(rs, ofs(v), st.x[v]);
      }
    }
    // RMSNorm: mean of squares.  LayerNorm: the mean, then the mean squared deviation
    // from it, both reduced from the registers (the row is read from memory once).
    // Deviations about the mean keep the variance exact for constant rows and free of
    // the cancellation of mean(x^2) - mean^2 when |mean| >> deviation.
    // Short rows keep the deviations from the mean for the output pass.
    constexpr bool KEEP = LN && VPL * EPV <= 32;
    float dev[KEEP ? VPL : 1][EPV];
    float mu = 0.0f, var;
    if constexpr (LN) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) s = D::sum(st.x[v], s);
      mu = row_sum(s, 0) * a.inv_n;
      float ss = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool in_row = v < VPL - 1 || last_in_row;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float d = in_row ? D::get(st.x[v], e) - mu : 0.0f;
          ss = fmaf(d, d, ss);
          if constexpr (KEEP) dev[v][e] = d;
        }
      }
      var = row_sum(ss, 1) * a.inv_n;
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) ss = D::sumsq(st.x[v], ss);
      var = row_sum(ss, 0) * a.inv_n;
    }
    if constexpr (WPR > 1) parity ^= 1;

    const float r = rsqrtf(var + a.eps);
    buf_stf(group_stat(a.rstd, grp), stat_ofs, r);
    if constexpr (LN) buf_stf(group_stat(a.mean, grp), stat_ofs, mu);

    const rsrc_t ry = group(a.y, grp);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      PV gv, bv;
      if constexpr (GREG) {
        gv = g[v];
        if constexpr (LN) bv = b[v];
      } else {
        gv.load_buf(rg, col_ofs(v));
        if constexpr (LN) bv.load_buf(rb, col_ofs(v));
      }
      float o[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        // Unpack the packed row afresh (or reuse the kept deviations), so that only
        // the packed words stay live across the reductions.
        if constexpr (LN) {
          const float d = KEEP ? dev[KEEP ? v : 0][e] : D::get_fresh(st.x[v], e) - mu;
          o[e] = fmaf(d * r, gv.get_fresh(e), bv.get_fresh(e));
        } else {
          o[e] = D::get_fresh(st.x[v], e) * r * gv.get_fresh(e);
        }
      }
      buf_st16(ry, ofs(v), D::pack(o));
    }
  };

  // Persistent loop over row groups b, b + G, b + 2G, ... through S stages of registers:
  // while one stage is reduced and stored, the loads of the next S - 1 groups are in
  // flight in the others.  The loop is unrolled S times so each stage keeps its
  // registers.  Loads for groups past the last read zeros through an empty resource and
  // are never used (the kernel is launched with several groups per workgroup, so these
  // few are a small part of its loads).
  int64_t grp = grp0;
  Stage st[S];
#pragma unroll
  for (int k = 0; k < S - 1; ++k) load(grp + k * G, st[k]);
  while (grp < gend) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
      // The scheduling barrier keeps these loads ahead of the work on the current stage
      // (otherwise the compiler moves that work up, and its wait for the current loads,
      // which is a wait for everything in flight before them, comes first).
      load(grp + (S - 1) * G, st[(k + S - 1) % S]);
      __builtin_amdgcn_sched_barrier(0);
      process(grp, st[k]);
      grp += G;
      if (k < S - 1 && grp >= gend) break;
    }
  }
}

// Row groups handed to one-group workgroups after the persistent ones, when every
// persistent workgroup still takes at least two groups (measured on MI355X: one per
// persistent workgroup gains 0.5-2 % over an even split).
inline int64_t fwd_tail_groups(int64_t groups, int grid) {
  return groups >= 3 * static_cast<int64_t>(grid) ? grid : 0;
}

template <bool LN, typename D, typename P, int LPR, int VPL>
hipError_t launch_one(const FwdArgs& a0, int grid, bool pipe, hipStream_t s) {
  if constexpr (VPL <= 8) {
    if (pipe && grid < a0.groups) {
      FwdArgs a = a0;
      if (const int64_t tail = fwd_tail_groups(a.groups, grid)) {
        a.persistent = grid;
        a.static_end = (a.groups - tail) / grid * grid;
        grid = static_cast<int>(grid + (a.groups - a.static_end));
      }
      if (a.res) {
        hipLaunchKernelGGL((fwd_pipe_kernel<LN, D, P, LPR, VPL, true, 2>), dim3(grid),
                           dim3(fwd_block(LPR)), 0, s, a);
      } else {
        hipLaunchKernelGGL((fwd_pipe_kernel<LN, D, P, LPR, VPL, false, 2>), dim3(grid),
                           dim3(fwd_block(LPR)), 0, s, a);
      }
      return hipGetLastError();
    }
  }
  if (a0.res) {
    hipLaunchKernelGGL((fwd_rows_kernel<LN, D, P, LPR, VPL, true>), dim3(grid),
                       dim3(fwd_block(LPR)), 0, s, a0);
  } else {
    hipLaunchKernelGGL((fwd_rows_kernel<LN, D, P, LPR, VPL, false>), dim3(grid),
                       dim3(fwd_block(LPR)), 0, s, a0);
  }
  return hipGetLastError();
}

}  // namespace

#define RN_CAT_(a, b, c, d) a##b##c##d
#define RN_CAT(a, b, c, d) RN_CAT_(a, b, c, d)
#define RN_LAUNCHER RN_CAT(launch_fwd_rows_k, RN_KIND, _t, RN_TC)

hipError_t RN_LAUNCHER(int lpr, int vpl, const FwdArgs& a, int grid, bool pipe, hipStream_t s) {
  constexpr bool kLN = RN_KIND == 1;
  using D = Types<RN_TC>::D;
  using P = Types<RN_TC>::P;
#define RN_CASE(L, V) \
  if (lpr == L && vpl == V) return launch_one<kLN, D, P, L, V>(a, grid, pipe, s);
  RN_FWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

}  // namespace rownorm
