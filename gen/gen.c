/*
 * Seeded synthetic inputs for the row-normalization tests and benchmark.
 *
 * This file holds no normalization arithmetic.  It only turns (seed, index)
 * into numbers: both the CPU oracle and the GPU library consume the bits it
 * writes, so the two sides always see identical inputs.
 *
 * Generator: a counter-based use of SplitMix64 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  Draw k of
 * stream s is mix64(s + (k + 1) * 0x9E3779B97F4A7C15), so any element can be
 * produced independently of the others and the result does not depend on the
 * number of threads.  Normal deviates come from the Box-Muller transform
 * (Box and Muller, 1958): draw k yields the pair (z0, z1) used for elements
 * 2k and 2k+1.
 *
 * Values are formed in double, rounded once to float, and, for bf16 or fp16
 * output, rounded again with round-to-nearest-even (NaN stays NaN; fp16 values
 * beyond its range become infinities).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GEN_F32 0
#define GEN_BF16 1
#define GEN_F16 2

static const uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t stream, uint64_t k) {
  return mix64(stream + (k + 1) * kGolden);
}

/* Open interval (0, 1) from 32 random bits. */
static inline double unit_open(uint32_t bits) {
  return ((double)bits + 0.5) * (1.0 / 4294967296.0);
}

/* [0, 1) from the top 53 bits. */
static inline double unit_53(uint64_t bits) {
  return (double)(bits >> 11) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign kept */
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* IEEE binary16 bits of a float, round-to-nearest-even. */
static inline uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
  if (a < 0x38800000u) {                                     /* below 2^-14: subnormal */
    float m;
    memcpy(&m, &a, 4);
    /* m * 2^24 is exact; rounding it to an integer (ties to even) gives the subnormal
     * significand, and 1024 is the smallest normal, encoded the same way. */
    return (uint16_t)(sign | (uint16_t)lrintf(m * 16777216.0f));
  }
  uint32_t h = ((a >> 23) - 112u) << 10 | ((a >> 13) & 0x3FFu); /* rebias 127 -> 15 */
  const uint32_t rem = a & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* may carry into the exponent */
  return (uint16_t)(sign | h);
}

/* Stream identifiers derived from the user seed, kept apart by a fixed odd
 * offset so that the normal stream and the outlier-mask stream never share
 * draws. */
static inline uint64_t normal_stream(uint64_t seed) { return mix64(seed); }
static inline uint64_t mask_stream(uint64_t seed) { return mix64(seed ^ 0xD1B54A32D192ED03ULL); }

static inline double normal_at(uint64_t stream, int64_t i) {
  uint64_t r = draw(stream, (uint64_t)(i >> 1));
  double u1 = unit_open((uint32_t)(r >> 32));
  double u2 = unit_open((uint32_t)r);
  double rad = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

/*
 * Fill out[0..n) with mean + std * z_i, where z_i ~ N(0,1).  When
 * outlier_p > 0, an independent Bernoulli(outlier_p) mask multiplies the
 * selected entries by outlier_scale (in float, before any bf16 rounding).
 * dtype: GEN_F32 writes float, GEN_BF16 / GEN_F16 write uint16 bfloat16 / binary16
 * bits.
 * Returns 0 on success, -1 on a bad argument.
 */
int gen_fill(void* out, int dtype, int64_t n, uint64_t seed, double mean, double std,
             double outlier_p, double outlier_scale) {
  if (n < 0 || (n > 0 && out == NULL) ||
      (dtype != GEN_F32 && dtype != GEN_BF16 && dtype != GEN_F16))
    return -1;
  const uint64_t ns = normal_stream(seed);
  const uint64_t ms = mask_stream(seed);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float v = (float)(mean + std * normal_at(ns, i));
    if (outlier_p > 0.0 && unit_53(draw(ms, (uint64_t)i)) < outlier_p) v = v * (float)outlier_scale;
    if (dtype == GEN_F32) {
      ((float*)out)[i] = v;
    } else if (dtype == GEN_BF16) {
      ((uint16_t*)out)[i] = f32_to_bf16_rne(v);
    } else {
      ((uint16_t*)out)[i] = f32_to_f16_rne(v);
    }
  }
  return 0;
}

/* Round float values to bfloat16 bits (RNE).  Used to hand identical bf16
 * bits to both sides when a test builds a tensor from explicit values. */
void gen_round_bf16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* Round float values to binary16 bits (RNE). */
void gen_round_f16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_rne(in[i]);
}
