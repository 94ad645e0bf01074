// The kernels outside the register-resident row mapping and the sliced passes
// (split_rows.hip):
//
//  * colreduce -- stage 2 of the two-stage dgamma/dbeta reduction: out[j] = sum over p of
//                part[p, j], in a fixed order (deterministic, no atomics; "Fused RMSNorm",
//                aryanashta.me, "What didn't work" and "Next").
//  * zero     -- clears dgamma/dbeta before the atomic comparison variants add into them.
//  * fwd_generic -- scalar forward for any N and alignment, for a call given no
//                workspace: a workgroup per row, one pass for the sums and a second
//                (cache-resident) pass to normalize.
//
// Formulas as in the forward and backward row kernels ("Fused RMSNorm", "What it is";
// "SOTA normalization performance with torch.compile", "How Did Torch.compile Catch
// Quack?" and "Why Is Peak Vectorization Your New Best Friend?").
#include <type_traits>

#include "launch.h"
#include "rownorm_dev.h"

namespace rownorm {
namespace {

constexpr int kRowWaves = kRowBlock / 64;

// Sum of two values over a kRowBlock-thread workgroup, identical in every thread.
// `red` holds 2 * kRowWaves * 2 floats, double-buffered by `parity`.
__device__ inline void block_sum2(float& a, float& b, float* red, int& parity) {
  a = group_sum<64>(a);
  b = group_sum<64>(b);
  const int wave = threadIdx.x >> 6;
  float* buf = red + parity * kRowWaves * 2;
  if ((threadIdx.x & 63) == 0) {
    buf[2 * wave] = a;
    buf[2 * wave + 1] = b;
  }
  __syncthreads();
  a = 0.0f;
  b = 0.0f;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    a += buf[2 * w];
    b += buf[2 * w + 1];
  }
  parity ^= 1;
}

// -------------------------------------------------------------------- colreduce
// S splits of the P rows x L = 256 / S lanes along N (4 columns each with 16-byte loads).
template <bool VEC4, int S>
__global__ __launch_bounds__(kColRedThreads) void colreduce_kernel(
    const float* __restrict__ part_g, const float* __restrict__ part_b, int64_t P, int32_t N,
    float* __restrict__ dgamma, float* __restrict__ dbeta) {
  constexpr int L = kColRedThreads / S;
  constexpr int W = VEC4 ? 4 : 1;
  const float* src = blockIdx.y ? part_b : part_g;
  float* dst = blockIdx.y ? dbeta : dgamma;
  const int tx = threadIdx.x % L;
  const int ty = threadIdx.x / L;
  const int64_t col = ((int64_t)blockIdx.x * L + tx) * W;
  // Split ty adds rows ty, ty + S, ty + 2S, ... in order; the S split sums are then added
  // in split order: a fixed order for a given P, so the result is reproducible bit for bit.
  float s[W];
#pragma unroll
  for (int k = 0; k < W; ++k) s[k] = 0.0f;
  if (col < N) {
#pragma unroll 4
    for (int64_t p = ty; p < P; p += S) {
      if constexpr (VEC4) {
        const float4 v = *reinterpret_cast<const float4*>(src + p * N + col);
        s[0] += v.x;
        s[1] += v.y;
        s[2] += v.z;
        s[3] += v.w;
      } else {
        s[0] += src[p * N + col];
      }
    }
  }
  __shared__ float buf[S][L * W];
#pragma unroll
  for (int k = 0; k < W; ++k) buf[ty][tx * W + k] = s[k];
  __syncthreads();
  // L * W columns per workgroup: up to four per thread when there is a single split
  for (int c = threadIdx.x; c < L * W; c += kColRedThreads) {
    const int64_t out = (int64_t)blockIdx.x * L * W + c;
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < S; ++q) t += buf[q][c];
    if (out < N) dst[out] = t;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* a, float* b, int32_t N) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < N; j += (int64_t)gridDim.x * 256) {
    a[j] = 0.0f;
    if (b) b[j] = 0.0f;
  }
}

// ------------------------------------------------------------------ fwd_generic
template <bool LN, typename D, typename P>
__global__ __launch_bounds__(kRowBlock) void fwd_generic_kernel(const FwdArgs a) {
  __shared__ float red[2 * kRowWaves * 2];
  int parity = 0;
  const int tid = threadIdx.x;
  // Element j of the row normalized: x, or with a fused residual add the sum x + res
  // rounded to the activation type (formed again on each pass, written on the last).
  auto elem = [&](int64_t i) {
    const float f = D::scalar(a.x, i);
    return a.res ? D::round(f + D::scalar(a.res, i)) : f;
  };
  for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x) {
    const int64_t base = row * a.N;
    // RMSNorm: mean of squares.  LayerNorm: mean, then mean squared deviation (a second,
    // cache-resident pass), as the register-resident kernel does.
    float mu = 0.0f, var;
    if constexpr (LN) {
      float s = 0.0f, unused = 0.0f;
#pragma unroll 4
      for (int64_t j = tid; j < a.N; j += kRowBlock) s += elem(base + j);
      block_sum2(s, unused, red, parity);
      mu = s * a.inv_n;
      float ss = 0.0f;
#pragma unroll 4
      for (int64_t j = tid; j < a.N; j += kRowBlock) {
        const float d = elem(base + j) - mu;
        ss = fmaf(d, d, ss);
      }
      block_sum2(ss, unused, red, parity);
      var = ss * a.inv_n;
    } else {
      float ss = 0.0f, unused = 0.0f;
#pragma unroll 4
      for (int64_t j = tid; j < a.N; j += kRowBlock) {
        const float f = elem(base + j);
        ss = fmaf(f, f, ss);
      }
      block_sum2(ss, unused, red, parity);
      var = ss * a.inv_n;
    }
    const float r = rsqrtf(var + a.eps);
    if (tid == 0) {
      if (a.rstd) a.rstd[row] = r;
      if constexpr (LN) {
        if (a.mean) a.mean[row] = mu;
      }
    }
#pragma unroll 4
    for (int64_t j = tid; j < a.N; j += kRowBlock) {
      const float f = elem(base + j);
      if (a.res) D::put_scalar(a.sum, base + j, f);
      const float gm = P::scalar(a.gamma, j);
      float o;
      if constexpr (LN) {
        o = fmaf((f - mu) * r, gm, P::scalar(a.beta, j));
      } else {
        o = f * r * gm;
      }
      D::put_scalar(a.y, base + j, o);
    }
  }
}

}  // namespace

// --------------------------------------------------------------------- launchers
// (kind, type pair) -> CALL(LayerNorm?, activation type, parameter type).
#define RN_DISPATCH_KT(kind, tc, CALL)                              \
  do {                                                              \
    const bool ln_ = kind == 1;                                     \
    if (tc == kTcF32) { if (ln_) CALL(true, F32, F32) else CALL(false, F32, F32) }       \
    if (tc == kTcBF16) { if (ln_) CALL(true, BF16, BF16) else CALL(false, BF16, BF16) }  \
    if (tc == kTcF16) { if (ln_) CALL(true, F16, F16) else CALL(false, F16, F16) }       \
    if (tc == kTcBF16F32) { if (ln_) CALL(true, BF16, F32) else CALL(false, BF16, F32) } \
    if (tc == kTcF16F32) { if (ln_) CALL(true, F16, F32) else CALL(false, F16, F32) }    \
  } while (0)

hipError_t launch_fwd_generic(int kind, int tc, const FwdArgs& a, int grid, hipStream_t s) {
#define RN_CALL(LN, D, P)                                                                    \
  {                                                                                         \
    hipLaunchKernelGGL((fwd_generic_kernel<LN, D, P>), dim3(grid), dim3(kRowBlock), 0, s, a); \
    return hipGetLastError();                                                               \
  }
  RN_DISPATCH_KT(kind, tc, RN_CALL);
#undef RN_CALL
  return hipErrorInvalidValue;
}

hipError_t launch_colreduce(const float* part_g, const float* part_b, int64_t P, int32_t N,
                            float* dgamma, float* dbeta, hipStream_t s) {
  const bool vec4 = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(part_g) & 15) == 0) &&
                    (part_b == nullptr || (reinterpret_cast<uintptr_t>(part_b) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(dgamma) & 15) == 0) &&
                    (dbeta == nullptr || (reinterpret_cast<uintptr_t>(dbeta) & 15) == 0);
  // As many splits of the P rows as there are rows, up to the most (a few partial rows
  // then leave no lanes idle); the rest of the 256 threads go along N.
  const int smax = colred_max_splits(vec4);
  int splits = 1;
  while (splits < smax && splits < P) splits *= 2;
  const int per_block = (kColRedThreads / splits) * (vec4 ? 4 : 1);
  const dim3 grid(static_cast<uint32_t>((static_cast<int64_t>(N) + per_block - 1) / per_block),
                  part_b ? 2 : 1);
#define RN_COLRED(V, S)                                                                     \
  if (vec4 == V && splits == S) {                                                           \
    hipLaunchKernelGGL((colreduce_kernel<V, S>), grid, dim3(kColRedThreads), 0, s, part_g,  \
                       part_b, P, N, dgamma, dbeta);                                        \
    return hipGetLastError();                                                               \
  }
  RN_COLRED(true, 1) RN_COLRED(true, 2) RN_COLRED(true, 4) RN_COLRED(true, 8)
  RN_COLRED(true, 16) RN_COLRED(true, 32)
  RN_COLRED(false, 1) RN_COLRED(false, 2) RN_COLRED(false, 4) RN_COLRED(false, 8)
#undef RN_COLRED
  return hipErrorInvalidValue;
}

// Streaming reference (a measurement aid, not on the normalization path): each workgroup
// owns a contiguous chunk of 256 x kStreamVecs 16-byte vectors, issues all its loads,
// then all its stores, with the norm kernels' non-temporal hints.  One vector per thread
// is the fastest form measured on MI355X (copy 6.5-6.6 TB/s and two reads + one write
// 6.4-6.5 TB/s over 256 MiB-1 GiB streams, against 6.1-6.25 with four per thread).
constexpr int kStreamVecs = 1;

template <bool TWO>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ a,
                                                     const u32x4* __restrict__ b,
                                                     u32x4* __restrict__ d, int64_t n) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * kStreamVecs + threadIdx.x;
  u32x4 r[kStreamVecs];
#pragma unroll
  for (int v = 0; v < kStreamVecs; ++v) {
    const int64_t i = base + v * 256;
    r[v] = i < n ? ld16_stream(a, i) : zero16();
    if constexpr (TWO) {
      if (i < n) r[v] += ld16_stream(b, i);
    }
  }
#pragma unroll
  for (int v = 0; v < kStreamVecs; ++v) {
    const int64_t i = base + v * 256;
    if (i < n) st16_stream(d, i, r[v]);
  }
}

hipError_t launch_stream_reference(bool two_reads, const void* a, const void* b, void* d,
                                   int64_t n, hipStream_t s) {
  const int64_t per_block = 256 * kStreamVecs;
  const int64_t grid = (n + per_block - 1) / per_block;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  u32x4* pd = static_cast<u32x4*>(d);
  if (two_reads) {
    hipLaunchKernelGGL((stream_kernel<true>), dim3(unsigned(grid)), dim3(256), 0, s, pa, pb, pd, n);
  } else {
    hipLaunchKernelGGL((stream_kernel<false>), dim3(unsigned(grid)), dim3(256), 0, s, pa, pb, pd,
                       n);
  }
  return hipGetLastError();
}

hipError_t launch_zero(float* a, float* b, int32_t N, hipStream_t s) {
  int64_t grid = (static_cast<int64_t>(N) + 255) / 256;
  if (grid > 1024) grid = 1024;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, a, b, N);
  return hipGetLastError();
}

}  // namespace rownorm
