/*
 * Seeded synthetic input generator (host C, OpenMP).
 *
 * This module only draws random numbers. It holds none of the MoE layer's
 * arithmetic: no routing, no dequantisation, no products. It serves both the
 * CPU oracle and the HIP library, so both see bit-identical inputs.
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator. Stream `key` yields word i = mix64(key + (i + 1) * GAMMA), which
 * is exactly the i-th output of a SplitMix64 generator seeded with `key`.
 * Because word i is a pure function of (key, i), any tensor, and any expert
 * inside a tensor, can be regenerated on its own and in parallel.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SM_GAMMA);
}

/* i-th SplitMix64 output of a generator seeded with `seed` (for pinning the
 * generator against the published sequence). */
uint64_t synth_splitmix64_at(uint64_t seed, uint64_t i) { return word_at(seed, i); }

/* Stream key for (seed, a, b, c, d): each field is absorbed through mix64 so
 * that nearby tuples give unrelated streams. */
uint64_t synth_key(uint64_t seed, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint64_t k = mix64(seed ^ 0x5EEDC0DE5EEDC0DEull);
  k = mix64(k ^ ((uint64_t)a << 32 | b));
  k = mix64(k ^ ((uint64_t)c << 32 | d) ^ 0xA5A5A5A5ull);
  return k;
}

/* Uniform double in (0, 1] from the top 53 bits. */
static inline double u01_open0(uint64_t w) { return ((double)(w >> 11) + 1.0) * 0x1.0p-53; }
/* Uniform double in [0, 1). */
static inline double u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

/* Standard normal for element i: Box-Muller on words 2i and 2i+1. */
static inline double normal_at(uint64_t key, int64_t i) {
  double u1 = u01_open0(word_at(key, 2 * (uint64_t)i));
  double u2 = u01(word_at(key, 2 * (uint64_t)i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* float -> bfloat16, round to nearest even (finite inputs only). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* float -> IEEE binary16, round to nearest even (finite inputs; overflow
 * saturates to infinity, tiny values become subnormal or zero). */
static inline uint16_t f32_to_f16_rne(float f) {
  uint32_t u = f32_bits(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  int32_t exp = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
  uint32_t man = u & 0x7FFFFFu;
  if (((u >> 23) & 0xFF) == 0) return (uint16_t)sign; /* f32 zero/subnormal */
  if (exp >= 31) return (uint16_t)(sign | 0x7C00u);
  if (exp <= 0) {
    if (exp < -10) return (uint16_t)sign;
    man |= 0x800000u;
    uint32_t shift = (uint32_t)(14 - exp);
    uint32_t half = 1u << (shift - 1);
    uint32_t rest = man & ((1u << shift) - 1);
    uint32_t r = man >> shift;
    if (rest > half || (rest == half && (r & 1u))) r++;
    return (uint16_t)(sign | r);
  }
  uint32_t r = man >> 13;
  uint32_t rest = man & 0x1FFFu;
  uint32_t out = ((uint32_t)exp << 10) | r;
  if (rest > 0x1000u || (rest == 0x1000u && (r & 1u))) out++; /* may carry into exponent: correct */
  return (uint16_t)(sign | out);
}

void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = f32_to_bf16_rne(in[i]);
}

/* N(mean, sd) rounded to float. */
void synth_normal_f32(uint64_t key, int64_t n, double mean, double sd, float *out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = (float)(mean + sd * normal_at(key, i));
}

/* N(0, sd) rounded to float, then to bfloat16 (RNE). */
void synth_normal_bf16(uint64_t key, int64_t n, double sd, uint16_t *out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = f32_to_bf16_rne((float)(sd * normal_at(key, i)));
}

/* U(lo, hi) rounded to float, then to binary16 (RNE). */
void synth_uniform_f16(uint64_t key, int64_t n, double lo, double hi, uint16_t *out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++)
    out[i] = f32_to_f16_rne((float)(lo + (hi - lo) * u01(word_at(key, (uint64_t)i))));
}

/* Signed integer codes uniform over [-2^(bits-1), 2^(bits-1) - 1], bits in
 * 1..8. Word w supplies the codes 8w .. 8w+7, one per byte, so a code is
 * the low `bits` bits of its byte, reinterpreted as two's complement. */
void synth_codes(uint64_t key, int64_t n, int bits, int8_t *out) {
  const int64_t nw = (n + 7) / 8;
  const uint32_t mask = (1u << bits) - 1u;
  const int32_t half = 1 << (bits - 1);
#pragma omp parallel for schedule(static) if (nw > 8192)
  for (int64_t w = 0; w < nw; w++) {
    uint64_t r = word_at(key, (uint64_t)w);
    for (int b = 0; b < 8; b++) {
      int64_t i = w * 8 + b;
      if (i < n) {
        int32_t v = (int32_t)((r >> (8 * b)) & mask);
        out[i] = (int8_t)(v >= half ? v - (1 << bits) : v);
      }
    }
  }
}

/* Uniform random permutation of 0..n-1 (Fisher-Yates, draws from the
 * stream in order; modulo bias is below 2^-40 for n < 2^24). */
void synth_permutation(uint64_t key, int32_t n, int32_t *out) {
  for (int32_t i = 0; i < n; i++) out[i] = i;
  for (int32_t i = n - 1; i > 0; i--) {
    uint64_t r = word_at(key, (uint64_t)(n - 1 - i));
    int32_t j = (int32_t)(r % (uint64_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}
