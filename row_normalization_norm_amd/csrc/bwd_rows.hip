// Backward kernel, register-resident rows (ROWS path), stage 1 of the two-stage
// dgamma/dbeta reduction.
//
// The backward's outputs are dx, dgamma and, for LayerNorm, dbeta, with reductions
// over dy ("SOTA normalization performance with torch.compile", theaicatchup.com,
// "Why Is Peak Vectorization Your New Best Friend?").  Per row, with the forward's
// saved statistics, xhat = (x - mean) * rstd (RMSNorm: x * rstd) and g = dy * gamma:
//     c1 = mean(g * xhat), c2 = mean(g) (LayerNorm only)
//     dx = rstd * (g - c2 - xhat * c1)
// and per column dgamma += dy * xhat, dbeta += dy.
//
// dx is computed the way the forward computes y: the rows of x and dy are loaded once
// into registers (16-byte loads), the two row sums are reduced across the row's lanes,
// and dx is written once.  The column sums stay in fp32 registers for every row the
// workgroup handles (for wide one-row workgroups in LDS, each lane owning its columns'
// words, which frees the registers for more resident waves); at the end the
// workgroup's row slots are combined in a fixed order and written as ONE partial row
// of a [P, N] workspace.  A separate
// column-reduce kernel then adds the P partial rows.  That is the atomic-free two-stage
// scheme the "Fused RMSNorm" page (aryanashta.me, "What didn't work") contrasts with
// atomically adding every block's partial into one shared vector; the atomic variants
// (per row, per workgroup) are kept for measurement only.
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

template <bool LN, typename D, typename P, int LPR, int VPL, bool ADD>
__global__ __launch_bounds__(bwd_block(LPR)) void bwd_rows_kernel(const BwdArgs a) {
  using PV = Param<D, P>;
  constexpr int BLOCK = bwd_block(LPR);
  constexpr int EPV = D::kPerVec;
  constexpr int ROWS = BLOCK / LPR;
  constexpr int WPR = LPR > 64 ? LPR / 64 : 1;

  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int slot = tid / LPR;
  const int nvec = a.nvec;
  const int mode = a.mode;

  // Per-column partial sums: registers, or (LACC) LDS words private to each lane, laid
  // out [dgamma|dbeta][vector][4-column chunk][lane] so that a wave's 16-byte accesses
  // are contiguous.
  constexpr bool LACC = bwd_lds_acc(LN, EPV, LPR, VPL);
  static_assert(!LACC || ROWS == 1, "LDS partials assume one row per workgroup");
  constexpr int CH = EPV / 4;
  constexpr int RV = LACC ? 1 : VPL;
  float accg[RV][EPV];
  float accb[LN ? RV : 1][EPV];
  __shared__ float4 lacc[LACC ? (LN ? 2 : 1) * VPL * CH * LPR : 1];
  auto lidx = [&](int which, int v, int h) { return ((which * VPL + v) * CH + h) * LPR + lane; };
  if constexpr (LACC) {
#pragma unroll
    for (int w = 0; w < (LN ? 2 : 1); ++w)
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int h = 0; h < CH; ++h) lacc[lidx(w, v, h)] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        accg[v][e] = 0.0f;
        if constexpr (LN) accb[v][e] = 0.0f;
      }
    }
  }

  __shared__ float red[WPR > 1 ? 2 * ROWS * WPR * 2 : 1];
  int parity = 0;

  // gamma stays in registers across the workgroup's rows when the row is short enough,
  // for the shortest rows also unpacked to fp32.
  constexpr bool GREG = VPL <= 2;
  constexpr bool GUNP = GREG && VPL * EPV <= 16;
  // Sums of dy * gamma straight from packed 16-bit words (dy and gamma of one type).
  constexpr bool kDot = !std::is_same<D, F32>::value && PV::kPacked;
  PV greg[GREG ? VPL : 1];
  float gunp[GUNP ? VPL : 1][EPV];
  if constexpr (GREG) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (vi < nvec) {
        greg[v].load(a.gamma, vi);
      } else {
        greg[v].clear();
      }
      if constexpr (GUNP) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) gunp[v][e] = greg[v].get(e);
      }
    }
  }

  // 1024-lane workgroups with 4 vectors per lane have no registers left for a second
  // row; their 16 waves per CU keep enough loads in flight without it.
  constexpr bool PF = !(LPR == 1024 && VPL > 2);
  constexpr bool OP = !PF;
  // The next row group's x, dy and saved statistics are loaded before the current one is
  // reduced, so HBM reads stay in flight through the reduction and the dx stores.
  // With ADD the gradient arriving at the residual sum comes with x and dy, and is
  // added to dx.
  auto load = [&](int64_t grp, u32x4 (&xb)[VPL], u32x4 (&db)[VPL], u32x4 (&gb)[ADD ? VPL : 1],
                  float& rb, float& mb) {
    const int64_t row = grp * ROWS + slot;
    const bool rok = row < a.M;
    if constexpr (OP) {
      // The widest mapping addresses the row from opaque per-lane pointers (no per-vector
      // 64-bit addresses hoisted out of the row loop).
      const int64_t lofs = row * nvec + lane;
      const u32x4* xp = opaque_ptr(static_cast<const u32x4*>(a.x) + lofs);
      const u32x4* dp = opaque_ptr(static_cast<const u32x4*>(a.dy) + lofs);
      const u32x4* rp = ADD ? opaque_ptr(static_cast<const u32x4*>(a.dres) + lofs) : nullptr;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool ok = rok && v * LPR + lane < nvec;
        xb[v] = ok ? ld16_stream(xp, v * LPR) : zero16();
        db[v] = ok ? ld16_stream(dp, v * LPR) : zero16();
        if constexpr (ADD) gb[v] = ok ? ld16_stream(rp, v * LPR) : zero16();
      }
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int vi = v * LPR + lane;
        const bool ok = rok && vi < nvec;
        xb[v] = ok ? ld16_stream(a.x, row * nvec + vi) : zero16();
        db[v] = ok ? ld16_stream(a.dy, row * nvec + vi) : zero16();
        if constexpr (ADD) gb[v] = ok ? ld16_stream(a.dres, row * nvec + vi) : zero16();
      }
    }
    rb = rok ? a.rstd[row] : 0.0f;
    mb = (LN && rok) ? a.mean[row] : 0.0f;
  };
  u32x4 nx[VPL], nd[VPL], ng[ADD ? VPL : 1];
  float nr = 0.0f, nmu = 0.0f;
  if (blockIdx.x < a.groups) load(blockIdx.x, nx, nd, ng, nr, nmu);

  for (int64_t grp = blockIdx.x; grp < a.groups; grp += gridDim.x) {
    const int64_t row = grp * ROWS + slot;
    const bool row_ok = row < a.M;
    const int64_t vbase = row * nvec;

    u32x4 xv[VPL], dv[VPL], rg[ADD ? VPL : 1];
    PV gv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      xv[v] = nx[v];
      dv[v] = nd[v];
      if constexpr (ADD) rg[v] = ng[v];
      if constexpr (GREG) {
        gv[v] = greg[v];
      } else if (row_ok && vi < nvec) {
        gv[v].load(a.gamma, vi);
      } else {
        gv[v].clear();
      }
    }
    const float r = nr;
    const float mu = nmu;
    if (PF && grp + gridDim.x < a.groups) load(grp + gridDim.x, nx, nd, ng, nr, nmu);

    // Row sums, and the per-column contributions (which do not need the row sums).
    // Short rows keep xhat and g in registers for the dx pass; longer ones unpack the
    // packed words again there, so that only those stay live across the reduction.
    constexpr bool KEEP = VPL * EPV <= 16;
    float kxh[KEEP ? VPL : 1][EPV], kg[KEEP ? VPL : 1][EPV];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      // LayerNorm's sum of g = dy * gamma: for 16-bit types straight from the packed words.
      if constexpr (LN && kDot) s2 = D::dot(dv[v], gv[v].v, s2);
      float xs[EPV], ds[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xh = (D::get(xv[v], e) - mu) * r;
        const float d = D::get(dv[v], e);
        const float g = d * (GUNP ? gunp[GUNP ? v : 0][e] : gv[v].get(e));
        s1 = fmaf(g, xh, s1);
        if constexpr (LN && !kDot) s2 += g;
        xs[e] = xh;
        ds[e] = d;
        if constexpr (!LACC) {
          accg[v][e] = fmaf(d, xh, accg[v][e]);
          if constexpr (LN) accb[v][e] += d;
        }
        if constexpr (KEEP) {
          kxh[v][e] = xh;
          kg[v][e] = g;
        }
      }
      if constexpr (LACC) {
        // Rows past M contribute zeros (x and dy load as zeros there).
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

    constexpr int W = LPR < 64 ? LPR : 64;
    s1 = group_sum<W>(s1);
    if constexpr (LN) s2 = group_sum<W>(s2);
    if constexpr (WPR > 1) {
      const int wave = (tid >> 6) % WPR;
      float* buf = red + (parity * ROWS + slot) * WPR * 2;
      if ((tid & 63) == 0) {
        buf[2 * wave] = s1;
        buf[2 * wave + 1] = s2;
      }
      __syncthreads();
      s1 = 0.0f;
      s2 = 0.0f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) {
        s1 += buf[2 * w];
        if constexpr (LN) s2 += buf[2 * w + 1];
      }
      parity ^= 1;
    }
    // dx = r * (g - c2 - xhat * c1) = g * r + (xhat * (-r * c1) + (-r * c2)).
    const float nrc1 = -r * (s1 * a.inv_n);
    const float nrc2 = LN ? -r * (s2 * a.inv_n) : 0.0f;

#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (row_ok && vi < nvec) {
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          float xh, g;
          if constexpr (KEEP) {
            xh = kxh[v][e];
            g = kg[v][e];
          } else {
            xh = (D::get_fresh(xv[v], e) - mu) * r;
            g = D::get_fresh(dv[v], e) * gv[v].get_fresh(e);
          }
          o[e] = fmaf(g, r, fmaf(xh, nrc1, nrc2));
          if constexpr (ADD) o[e] += D::get_fresh(rg[v], e);
        }
        st16_stream(a.dx, vbase + vi, D::pack(o));
        if (mode == kAtomicRow) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const int col = vi * EPV + e;
            const float d = D::get_fresh(dv[v], e);
            unsafeAtomicAdd(a.dgamma + col, d * ((D::get_fresh(xv[v], e) - mu) * r));
            if constexpr (LN) unsafeAtomicAdd(a.dbeta + col, d);
          }
        }
      }
    }
    if (!PF && grp + gridDim.x < a.groups) load(grp + gridDim.x, nx, nd, ng, nr, nmu);
  }

  if (mode == kAtomicRow) return;

  // Combine the workgroup's row slots and emit one partial row (or, in the per-workgroup
  // atomic mode, add it into dgamma/dbeta).
  float* const out_g = mode == kTwoStage ? a.part_g + (int64_t)blockIdx.x * a.N : a.dgamma;
  float* const out_b = mode == kTwoStage ? a.part_b + (int64_t)blockIdx.x * a.N : a.dbeta;
  if constexpr (LACC) {
    // Each lane reads back only the LDS words it wrote: no barrier is needed.
#pragma unroll
    for (int w = 0; w < (LN ? 2 : 1); ++w) {
      float* const out = w == 0 ? out_g : out_b;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int vi = v * LPR + lane;
        if (vi < nvec) {
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            const float4 t = lacc[lidx(w, v, h)];
            const int col = vi * EPV + 4 * h;
            if (mode == kTwoStage) {
              *reinterpret_cast<float4*>(out + col) = t;
            } else {
              unsafeAtomicAdd(out + col, t.x);
              unsafeAtomicAdd(out + col + 1, t.y);
              unsafeAtomicAdd(out + col + 2, t.z);
              unsafeAtomicAdd(out + col + 3, t.w);
            }
          }
        }
      }
    }
  } else if constexpr (ROWS == 1) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (vi < nvec) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int col = vi * EPV + e;
          if (mode == kTwoStage) {
            out_g[col] = accg[v][e];
            if constexpr (LN) out_b[col] = accb[v][e];
          } else {
            unsafeAtomicAdd(out_g + col, accg[v][e]);
            if constexpr (LN) unsafeAtomicAdd(out_b + col, accb[v][e]);
          }
        }
      }
    }
  } else {
    // cbuf holds one vector column block of every slot: element e of lane l of a slot at
    // l*(EPV+1) + e.  The pad word keeps the lanes' stores, EPV words apart otherwise, on
    // distinct LDS banks.
    constexpr int SPAN = LPR * EPV;
    constexpr int PSPAN = LPR * (EPV + 1);
    __shared__ float cbuf[ROWS * PSPAN];
#pragma unroll
    for (int pass = 0; pass < (LN ? 2 : 1); ++pass) {
      float* const out = pass == 0 ? out_g : out_b;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          cbuf[slot * PSPAN + lane * (EPV + 1) + e] = pass == 0 ? accg[v][e] : accb[LN ? v : 0][e];
        }
        __syncthreads();
        for (int c = tid; c < SPAN; c += BLOCK) {
          float sum = 0.0f;
#pragma unroll 4
          for (int k = 0; k < ROWS; ++k) sum += cbuf[k * PSPAN + (c / EPV) * (EPV + 1) + c % EPV];
          const int col = v * SPAN + c;
          if (col < a.N) {
            if (mode == kTwoStage) {
              out[col] = sum;
            } else {
              unsafeAtomicAdd(out + col, sum);
            }
          }
        }
      }
    }
  }
}

// Pipelined backward for persistent grids (several row groups per workgroup) in the
// two-stage mode.  The same computation as bwd_rows_kernel, with every access to x, dy,
// dx, the residual gradient, the saved statistics and gamma a raw buffer access through a
// resource of the row group (ROWS consecutive rows; groups past the last row get an empty
// one) or of gamma, so that none sits under a branch: rows past M and the padding lanes of
// the last vector slot read zeros (and so add nothing to the column sums) and drop their
// stores.  The row loop is unrolled twice over two fixed sets of registers, the next
// group's loads issued into one while the other is reduced and stored.  The compiler can
// then count the memory operations in flight and wait only for the loads a step uses; the
// plain kernel's loop waited for every load and store, its own dx stores included, at the
// end of each iteration.
template <bool LN, typename D, typename P, int LPR, int VPL, bool ADD>
__global__ __launch_bounds__(bwd_block(LPR)) void bwd_pipe_kernel(const BwdArgs a) {
  using PV = Param<D, P>;
  constexpr int BLOCK = bwd_block(LPR);
  constexpr int EPV = D::kPerVec;
  constexpr int ROWS = BLOCK / LPR;
  constexpr int WPR = LPR > 64 ? LPR / 64 : 1;

  const int tid = threadIdx.x;
  const int lane = tid % LPR;
  const int slot = tid / LPR;
  const int nvec = a.nvec;
  const uint32_t row_bytes = static_cast<uint32_t>(nvec) * 16u;

  // Byte offset of this lane's vector slot v inside its row group (col_ofs: inside the
  // row, for gamma).  Only the last slot can hold padding lanes; they get an
  // out-of-range offset.
  const bool last_in_row = (VPL - 1) * LPR + lane < nvec;
  const uint32_t row_ofs = static_cast<uint32_t>(slot) * row_bytes;
  auto col_ofs = [&](int v) -> uint32_t {
    return (v == VPL - 1 && !last_in_row) ? kOutOfRange
                                          : static_cast<uint32_t>(v * LPR + lane) * 16u;
  };
  auto ofs = [&](int v) -> uint32_t {
    return (v == VPL - 1 && !last_in_row) ? kOutOfRange
                                          : row_ofs + static_cast<uint32_t>(v * LPR + lane) * 16u;
  };
  auto group_rows = [&](int64_t grp) -> uint32_t {
    const int64_t left = a.M - grp * ROWS;
    return left <= 0 ? 0u : left >= ROWS ? uint32_t(ROWS) : static_cast<uint32_t>(left);
  };
  auto group = [&](const void* base, int64_t grp) {
    return make_rsrc(static_cast<const char*>(base) + grp * ROWS * static_cast<int64_t>(row_bytes),
                     group_rows(grp) * row_bytes);
  };
  auto group_stat = [&](const float* base, int64_t grp) {
    return make_rsrc(base + grp * ROWS, group_rows(grp) * 4u);
  };
  const uint32_t stat_ofs = static_cast<uint32_t>(slot) * 4u;

  // Per-column partial sums: registers, or (LACC) LDS words private to each lane, laid
  // out [dgamma|dbeta][vector][4-column chunk][lane] so that a wave's 16-byte accesses
  // are contiguous.
  constexpr bool LACC = bwd_lds_acc(LN, EPV, LPR, VPL);
  static_assert(!LACC || ROWS == 1, "LDS partials assume one row per workgroup");
  constexpr int CH = EPV / 4;
  constexpr int RV = LACC ? 1 : VPL;
  float accg[RV][EPV];
  float accb[LN ? RV : 1][EPV];
  __shared__ float4 lacc[LACC ? (LN ? 2 : 1) * VPL * CH * LPR : 1];
  auto lidx = [&](int which, int v, int h) { return ((which * VPL + v) * CH + h) * LPR + lane; };
  if constexpr (LACC) {
#pragma unroll
    for (int w = 0; w < (LN ? 2 : 1); ++w)
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int h = 0; h < CH; ++h) lacc[lidx(w, v, h)] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        accg[v][e] = 0.0f;
        if constexpr (LN) accb[v][e] = 0.0f;
      }
    }
  }

  __shared__ float red[WPR > 1 ? 2 * ROWS * WPR * 2 : 1];
  int parity = 0;

  // gamma stays in registers across the workgroup's rows when the row is short enough,
  // for the shortest rows also unpacked to fp32.
  constexpr bool GREG = VPL <= 2;
  constexpr bool GUNP = GREG && VPL * EPV <= 16;
  constexpr bool kDot = !std::is_same<D, F32>::value && PV::kPacked;
  constexpr int kPB = PV::kPacked ? 16 : 32;
  const rsrc_t rgam = make_rsrc(a.gamma, static_cast<uint32_t>(nvec) * kPB);
  PV greg[GREG ? VPL : 1];
  float gunp[GUNP ? VPL : 1][EPV];
  if constexpr (GREG) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      greg[v].load_buf(rgam, col_ofs(v));
      if constexpr (GUNP) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) gunp[v][e] = greg[v].get(e);
      }
    }
  }

  struct Stage {
    u32x4 x[VPL], d[VPL];
    u32x4 g2[ADD ? VPL : 1];  // ADD: the gradient arriving at the residual sum
    float r, mu;
  };
  auto load = [&](int64_t grp, Stage& st) {
    const rsrc_t rx = group(a.x, grp), rd = group(a.dy, grp);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      st.x[v] = buf_ld16(rx, ofs(v));
      st.d[v] = buf_ld16(rd, ofs(v));
    }
    if constexpr (ADD) {
      const rsrc_t rr = group(a.dres, grp);
#pragma unroll
      for (int v = 0; v < VPL; ++v) st.g2[v] = buf_ld16(rr, ofs(v));
    }
    st.r = buf_ldf(group_stat(a.rstd, grp), stat_ofs);
    st.mu = LN ? buf_ldf(group_stat(a.mean, grp), stat_ofs) : 0.0f;
  };

  auto process = [&](int64_t grp, Stage& st) {
    PV gv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if constexpr (GREG) {
        gv[v] = greg[v];
      } else {
        gv[v].load_buf(rgam, col_ofs(v));
      }
    }
    const float r = st.r;
    const float mu = st.mu;

    // Row sums, and the per-column contributions (which do not need the row sums).
    // Short rows keep xhat and g in registers for the dx pass; longer ones unpack the
    // packed words again there, so that only those stay live across the reduction.
    constexpr bool KEEP = VPL * EPV <= 16;
    float kxh[KEEP ? VPL : 1][EPV], kg[KEEP ? VPL : 1][EPV];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if constexpr (LN && kDot) s2 = D::dot(st.d[v], gv[v].v, s2);
      float xs[EPV], ds[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xh = (D::get(st.x[v], e) - mu) * r;
        const float d = D::get(st.d[v], e);
        const float g = d * (GUNP ? gunp[GUNP ? v : 0][e] : gv[v].get(e));
        s1 = fmaf(g, xh, s1);
        if constexpr (LN && !kDot) s2 += g;
        xs[e] = xh;
        ds[e] = d;
        if constexpr (!LACC) {
          accg[v][e] = fmaf(d, xh, accg[v][e]);
          if constexpr (LN) accb[v][e] += d;
        }
        if constexpr (KEEP) {
          kxh[v][e] = xh;
          kg[v][e] = g;
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

    constexpr int W = LPR < 64 ? LPR : 64;
    s1 = group_sum<W>(s1);
    if constexpr (LN) s2 = group_sum<W>(s2);
    if constexpr (WPR > 1) {
      const int wave = (tid >> 6) % WPR;
      float* buf = red + (parity * ROWS + slot) * WPR * 2;
      if ((tid & 63) == 0) {
        buf[2 * wave] = s1;
        buf[2 * wave + 1] = s2;
      }
      __syncthreads();
      s1 = 0.0f;
      s2 = 0.0f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) {
        s1 += buf[2 * w];
        if constexpr (LN) s2 += buf[2 * w + 1];
      }
      parity ^= 1;
    }
    // dx = r * (g - c2 - xhat * c1) = g * r + (xhat * (-r * c1) + (-r * c2)).
    const float nrc1 = -r * (s1 * a.inv_n);
    const float nrc2 = LN ? -r * (s2 * a.inv_n) : 0.0f;

    const rsrc_t rdx = group(a.dx, grp);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      float o[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        float xh, g;
        if constexpr (KEEP) {
          xh = kxh[v][e];
          g = kg[v][e];
        } else {
          xh = (D::get_fresh(st.x[v], e) - mu) * r;
          g = D::get_fresh(st.d[v], e) * gv[v].get_fresh(e);
        }
        o[e] = fmaf(g, r, fmaf(xh, nrc1, nrc2));
        if constexpr (ADD) o[e] += D::get_fresh(st.g2[v], e);
      }
      buf_st16(rdx, ofs(v), D::pack(o));
    }
  };

  // Persistent loop over row groups b, b + G, b + 2G, ... in pairs of stages.  Loads for
  // groups past the last read zeros through an empty resource and are never used (the
  // kernel is launched with several groups per workgroup).
  const int64_t G = gridDim.x;
  int64_t grp = blockIdx.x;
  {
    Stage A, B;
    load(grp, A);
    while (grp < a.groups) {
      // The scheduling barriers keep the next group's loads ahead of the work on the
      // current one (otherwise the compiler moves that work up, and its wait for the
      // current loads, which is a wait for everything in flight before them, comes
      // first).
      load(grp + G, B);
      __builtin_amdgcn_sched_barrier(0);
      process(grp, A);
      grp += G;
      if (grp >= a.groups) break;
      load(grp + G, A);
      __builtin_amdgcn_sched_barrier(0);
      process(grp, B);
      grp += G;
    }
  }

  // Combine the workgroup's row slots and emit one partial row.
  float* const out_g = a.part_g + (int64_t)blockIdx.x * a.N;
  float* const out_b = a.part_b + (int64_t)blockIdx.x * a.N;
  if constexpr (LACC) {
    // Each lane reads back only the LDS words it wrote: no barrier is needed.
#pragma unroll
    for (int w = 0; w < (LN ? 2 : 1); ++w) {
      float* const out = w == 0 ? out_g : out_b;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int vi = v * LPR + lane;
        if (vi < nvec) {
#pragma unroll
          for (int h = 0; h < CH; ++h)
            *reinterpret_cast<float4*>(out + vi * EPV + 4 * h) = lacc[lidx(w, v, h)];
        }
      }
    }
  } else if constexpr (ROWS == 1) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * LPR + lane;
      if (vi < nvec) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int col = vi * EPV + e;
          out_g[col] = accg[v][e];
          if constexpr (LN) out_b[col] = accb[v][e];
        }
      }
    }
  } else {
    // cbuf holds one vector column block of every slot: element e of lane l of a slot at
    // l*(EPV+1) + e.  The pad word keeps the lanes' stores, EPV words apart otherwise, on
    // distinct LDS banks.
    constexpr int SPAN = LPR * EPV;
    constexpr int PSPAN = LPR * (EPV + 1);
    __shared__ float cbuf[ROWS * PSPAN];
#pragma unroll
    for (int pass = 0; pass < (LN ? 2 : 1); ++pass) {
      float* const out = pass == 0 ? out_g : out_b;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          cbuf[slot * PSPAN + lane * (EPV + 1) + e] = pass == 0 ? accg[v][e] : accb[LN ? v : 0][e];
        }
        __syncthreads();
        for (int c = tid; c < SPAN; c += BLOCK) {
          float sum = 0.0f;
#pragma unroll 4
          for (int k = 0; k < ROWS; ++k) sum += cbuf[k * PSPAN + (c / EPV) * (EPV + 1) + c % EPV];
          const int col = v * SPAN + c;
          if (col < a.N) out[col] = sum;
        }
      }
    }
  }
}

template <bool LN, typename D, typename P, int LPR, int VPL>
hipError_t launch_one(const BwdArgs& a, int grid, bool pipe, hipStream_t s) {
  // The pipelined kernel when asked for on a persistent grid in the two-stage mode (the
  // 1024-lane mappings of 4 vectors have no registers for a second stage).
  if constexpr (!(LPR == 1024 && VPL > 2)) {
    if (pipe && a.mode == kTwoStage && grid < a.groups) {
      if (a.dres) {
        hipLaunchKernelGGL((bwd_pipe_kernel<LN, D, P, LPR, VPL, true>), dim3(grid),
                           dim3(bwd_block(LPR)), 0, s, a);
      } else {
        hipLaunchKernelGGL((bwd_pipe_kernel<LN, D, P, LPR, VPL, false>), dim3(grid),
                           dim3(bwd_block(LPR)), 0, s, a);
      }
      return hipGetLastError();
    }
  }
  if (a.dres) {
    hipLaunchKernelGGL((bwd_rows_kernel<LN, D, P, LPR, VPL, true>), dim3(grid),
                       dim3(bwd_block(LPR)), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_rows_kernel<LN, D, P, LPR, VPL, false>), dim3(grid),
                       dim3(bwd_block(LPR)), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

#define RN_CAT_(a, b, c, d) a##b##c##d
#define RN_CAT(a, b, c, d) RN_CAT_(a, b, c, d)
#define RN_LAUNCHER RN_CAT(launch_bwd_rows_k, RN_KIND, _t, RN_TC)

hipError_t RN_LAUNCHER(int lpr, int vpl, const BwdArgs& a, int grid, bool pipe, hipStream_t s) {
  constexpr bool kLN = RN_KIND == 1;
  using D = Types<RN_TC>::D;
  using P = Types<RN_TC>::P;
#define RN_CASE(L, V)                                                \
  if constexpr (bwd_mapping_built(kLN, D::kPerVec, L, V)) {          \
    if (lpr == L && vpl == V) return launch_one<kLN, D, P, L, V>(a, grid, pipe, s); \
  }
  RN_BWD_MAPPINGS(RN_CASE)
#undef RN_CASE
  return hipErrorInvalidValue;
}

}  // namespace rownorm
