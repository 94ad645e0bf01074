// Device primitives for the row-normalization kernels (gfx950, wave64).
//
//  * 16-byte vector loads and stores (one global_load/store_dwordx4 per lane);
//  * bf16 <-> fp32: widening is exact (bf16 bits are the top half of an fp32);
//    narrowing uses v_cvt_pk_bf16_f32 (round to nearest even, NaN stays NaN);
//  * fp16 <-> fp32: widening is exact (v_cvt_f32_f16, or folded into v_fma_mix_f32 by
//    the compiler); narrowing uses v_cvt_pk_f16_f32 (round to nearest even);
//  * sums over aligned groups of 2..64 lanes with DPP (quad_perm, row_half_mirror,
//    row_mirror) inside a 16-lane row and lane shuffles across rows.  Every lane of a
//    group ends with the same bits, because each step adds the same two operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rownorm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element types
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static inline float get(const u32x4& v, int e) { return __uint_as_float(v[e]); }
  __device__ static inline float get_fresh(const u32x4& v, int e) { return __uint_as_float(v[e]); }
  __device__ static inline float scalar(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void put_scalar(void* p, int64_t i, float f) {
    static_cast<float*>(p)[i] = f;
  }
  // Sum and sum of squares of the vector's elements added to acc.
  __device__ static inline float sum(const u32x4& v, float acc) {
    return acc + ((get(v, 0) + get(v, 1)) + (get(v, 2) + get(v, 3)));
  }
  __device__ static inline float sumsq(const u32x4& v, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(get(v, e), get(v, e), acc);
    return acc;
  }
  __device__ static inline float dot(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(get(a, e), get(b, e), acc);
    return acc;
  }
  // a + b element by element, rounded to this type (the residual sum).
  __device__ static inline u32x4 add(const u32x4& a, const u32x4& b) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(get(a, e) + get(b, e));
    return r;
  }
  __device__ static inline float round(float f) { return f; }
  __device__ static inline u32x4 pack(const float (&f)[4]) {
    u32x4 r;
    r[0] = __float_as_uint(f[0]);
    r[1] = __float_as_uint(f[1]);
    r[2] = __float_as_uint(f[2]);
    r[3] = __float_as_uint(f[3]);
    return r;
  }
};

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  // Element e of the vector lives in 32-bit word e/2: low half for even e.
  __device__ static inline float get(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  // Same value as get(), through an opaque instruction: the compiler can neither merge
  // it with an earlier unpack nor hoist it out of a loop, so only the packed words have
  // to stay live in registers between two uses of a row.
  __device__ static inline float get_fresh(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    uint32_t r;
    if (e & 1) {
      asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(r) : "v"(w));
    } else {
      asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(w));
    }
    return __uint_as_float(r);
  }
  __device__ static inline float scalar(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  // Sum and sum of squares straight from the packed words with the bf16 dot product
  // (v_dot2_f32_bf16: two exact bf16 products added to an fp32 accumulator), so the
  // reductions need no unpacking.  The word goes through a local copy: a direct bit
  // cast of the extracted vector element to bf16x2 has been seen to make hipcc read
  // the same word four times.
  __device__ static inline bf16x2 word(const u32x4& v, int w) {
    const uint32_t u = v[w];
    bf16x2 h;
    __builtin_memcpy(&h, &u, sizeof(h));
    return h;
  }
  __device__ static inline float sum(const u32x4& v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(word(v, w), one, acc, false);
    return acc;
  }
  __device__ static inline float sumsq(const u32x4& v, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 h = word(v, w);
      acc = __builtin_amdgcn_fdot2_f32_bf16(h, h, acc, false);
    }
    return acc;
  }
  // acc + sum_e a_e * b_e.
  __device__ static inline float dot(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(word(a, w), word(b, w), acc, false);
    return acc;
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  __device__ static inline void put_scalar(void* p, int64_t i, float f) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack2(f, 0.0f) & 0xFFFFu);
  }
  __device__ static inline float round(float f) { return __uint_as_float(pack2(0.0f, f) & 0xFFFF0000u); }
  __device__ static inline u32x4 pack(const float (&f)[8]) {
    u32x4 r;
    r[0] = pack2(f[0], f[1]);
    r[1] = pack2(f[2], f[3]);
    r[2] = pack2(f[4], f[5]);
    r[3] = pack2(f[6], f[7]);
    return r;
  }
  // a + b element by element in fp32, rounded to this type (the residual sum).
  __device__ static inline u32x4 add(const u32x4& a, const u32x4& b) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = get(a, e) + get(b, e);
    return pack(f);
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  // Element e of the vector lives in 32-bit word e/2: low half for even e.
  __device__ static inline float get(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    return static_cast<float>(
        __builtin_bit_cast(_Float16, static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu))));
  }
  // Same value as get(), through an opaque instruction (see BF16::get_fresh).
  __device__ static inline float get_fresh(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    float r;
    if (e & 1) {
      asm volatile("v_cvt_f32_f16_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1"
                   : "=v"(r)
                   : "v"(w));
    } else {
      asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(r) : "v"(w));
    }
    return r;
  }
  __device__ static inline float scalar(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
  __device__ static inline void put_scalar(void* p, int64_t i, float f) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(f);
  }
  __device__ static inline float round(float f) { return static_cast<float>(static_cast<_Float16>(f)); }
  __device__ static inline f16x2 word(const u32x4& v, int w) {
    const uint32_t u = v[w];
    f16x2 h;
    __builtin_memcpy(&h, &u, sizeof(h));
    return h;
  }
  // Sum, sum of squares and dot product from the packed words (v_dot2_f32_f16: two exact
  // fp16 products added to an fp32 accumulator).
  __device__ static inline float sum(const u32x4& v, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2(word(v, w), one, acc, false);
    return acc;
  }
  __device__ static inline float sumsq(const u32x4& v, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f16x2 h = word(v, w);
      acc = __builtin_amdgcn_fdot2(h, h, acc, false);
    }
    return acc;
  }
  __device__ static inline float dot(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2(word(a, w), word(b, w), acc, false);
    return acc;
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
  __device__ static inline u32x4 pack(const float (&f)[8]) {
    u32x4 r;
    r[0] = pack2(f[0], f[1]);
    r[1] = pack2(f[2], f[3]);
    r[2] = pack2(f[4], f[5]);
    r[3] = pack2(f[6], f[7]);
    return r;
  }
  // a + b element by element in fp32, rounded to this type (the residual sum).
  __device__ static inline u32x4 add(const u32x4& a, const u32x4& b) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = get(a, e) + get(b, e);
    return pack(f);
  }
};

// The (activation, parameter) type pairs the kernels are built for, numbered as in
// launch.h's TypeCombo: fp32/fp32, bf16/bf16, fp16/fp16, bf16/fp32, fp16/fp32.
template <int TC> struct Types;
template <> struct Types<0> { using D = F32; using P = F32; };
template <> struct Types<1> { using D = BF16; using P = BF16; };
template <> struct Types<2> { using D = F16; using P = F16; };
template <> struct Types<3> { using D = BF16; using P = F32; };
template <> struct Types<4> { using D = F16; using P = F32; };

// ------------------------------------------------------------------ vector memory
__device__ inline u32x4 ld16(const void* base, int64_t vec_index) {
  return static_cast<const u32x4*>(base)[vec_index];
}
__device__ inline void st16(void* base, int64_t vec_index, const u32x4& v) {
  static_cast<u32x4*>(base)[vec_index] = v;
}
// The same pointer, opaque to the optimiser: addresses formed from it inside a loop are
// not hoisted out of the loop as one live 64-bit address per vector (which spills the
// widest mappings).  It passes through the empty asm as a global (address space 1)
// pointer, so the loads made through it are global loads: a flat load would also count
// against the LDS wait counter, and every later LDS access would then wait for the row's
// HBM reads.
template <typename T>
__device__ inline T* opaque_ptr(T* p) {
  auto g = (__attribute__((address_space(1))) T*)p;
  asm volatile("" : "+v"(g));
  return (T*)g;
}

// Streaming variants for data touched once (x, dy, y, dx): non-temporal hint, so the
// stream does not evict gamma/beta and the partial rows from the caches.
__device__ inline u32x4 ld16_stream(const void* base, int64_t vec_index) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(base) + vec_index);
}
__device__ inline void st16_stream(void* base, int64_t vec_index, const u32x4& v) {
  __builtin_nontemporal_store(v, static_cast<u32x4*>(base) + vec_index);
}

// Raw buffer access (CDNA buffer resource: 48-bit base, byte size, no stride).  A load at
// or past the end reads zero and a store there is dropped, by the hardware's range check,
// so ragged slices and rows past the last need no branch around the access.  Without
// branches the compiler can count the loads still in flight exactly and wait for just
// the ones a computation needs (a load under a branch makes it wait for all of them).
// The resource has to be uniform across the workgroup (it lives in scalar registers).
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit data, the GFX9-family encoding
constexpr int kBufferNT = 2;              // non-temporal cache policy (GFX940 family)
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferFlags);
}
__device__ inline u32x4 buf_ld16(rsrc_t r, uint32_t byte_ofs) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_ofs, 0, kBufferNT);
}
__device__ inline void buf_st16(rsrc_t r, uint32_t byte_ofs, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_ofs, 0, kBufferNT);
}
__device__ inline float buf_ldf(rsrc_t r, uint32_t byte_ofs) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_ofs, 0, 0));
}
__device__ inline void buf_stf(rsrc_t r, uint32_t byte_ofs, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_ofs, 0, 0);
}
// Cached (temporal) 16-byte load, for data every workgroup reads (gamma, beta).
__device__ inline u32x4 buf_ld16_cached(rsrc_t r, uint32_t byte_ofs) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_ofs, 0, 0);
}
// A byte offset that no buffer the kernels address reaches (every resource they build
// is smaller than 1 GiB), so an access made with it reads zero or is dropped; twice it,
// the offset of the second half of a pair of vectors, still is out of range.
constexpr uint32_t kOutOfRange = 0x40000000u;

__device__ inline u32x4 zero16() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// ------------------------------------------------------------- gamma and beta
// The EPV parameters (gamma or beta) that go with one 16-byte vector of activations of
// type D, stored as type P: one 16-byte vector when P is D, two when fp32 parameters go
// with 16-bit activations (EPV = 8).
template <typename D, typename P, bool kSame = std::is_same<D, P>::value>
struct Param;

template <typename D, typename P>
struct Param<D, P, true> {
  static constexpr bool kPacked = true;  // the same packing as the activations
  u32x4 v;
  __device__ inline void load(const void* base, int64_t vi) { v = ld16(base, vi); }
  // From a buffer resource of the parameters, at the byte offset of the activation
  // vector they go with (kOutOfRange: zeros).
  __device__ inline void load_buf(rsrc_t r, uint32_t act_ofs) { v = buf_ld16_cached(r, act_ofs); }
  __device__ inline void clear() { v = zero16(); }
  __device__ inline float get(int e) const { return D::get(v, e); }
  __device__ inline float get_fresh(int e) const { return D::get_fresh(v, e); }
};

template <typename D, typename P>
struct Param<D, P, false> {
  static_assert(std::is_same<P, F32>::value && D::kPerVec == 8,
                "mixed precision pairs 16-bit activations with fp32 parameters");
  static constexpr bool kPacked = false;
  u32x4 v[2];
  __device__ inline void load(const void* base, int64_t vi) {
    v[0] = ld16(base, 2 * vi);
    v[1] = ld16(base, 2 * vi + 1);
  }
  // fp32 parameters take twice the activations' bytes: byte offset 2 * act_ofs.
  __device__ inline void load_buf(rsrc_t r, uint32_t act_ofs) {
    v[0] = buf_ld16_cached(r, 2u * act_ofs);
    v[1] = buf_ld16_cached(r, 2u * act_ofs + 16u);
  }
  __device__ inline void clear() {
    v[0] = zero16();
    v[1] = zero16();
  }
  __device__ inline float get(int e) const { return __uint_as_float(v[e >> 2][e & 3]); }
  __device__ inline float get_fresh(int e) const { return get(e); }
};

// ------------------------------------------------------------------- reductions
// DPP control codes (GFX9): quad_perm selectors, and the row mirrors.
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm:[1,0,3,2]  (lane ^ 1)
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm:[2,3,0,1]  (lane ^ 2)
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each 16 lanes

template <int kCtrl>
__device__ inline float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

// Sum over aligned groups of W consecutive lanes (W a power of two, 1..64); the result
// is in every lane of the group.  Needs every lane of the wavefront to execute it.
template <int W>
__device__ inline float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v = dpp_add<kDppQuadSwap1>(v);
  if constexpr (W >= 4) v = dpp_add<kDppQuadSwap2>(v);
  if constexpr (W >= 8) v = dpp_add<kDppRowHalfMirror>(v);
  if constexpr (W >= 16) v = dpp_add<kDppRowMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace rownorm
