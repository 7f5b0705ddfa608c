// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// dot2 of bf16 pairs with fp32 accumulate: c + a.lo*b.lo + a.hi*b.hi
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Code extraction. A "pair" is a 32-bit register holding two 16-bit floats
// built with a magic exponent: with MAGIC = 0x4300 (bf16 128.0) the halves
// are bf16(128 + code); with MAGIC = 0x6400 (fp16 1024.0) they are
// fp16(1024 + code). Codes are the unsigned stored values (signed + 8 for
// Q4, signed + 4 for Q3). Pair i holds chunk elements 2i (low) and 2i+1.
// ---------------------------------------------------------------------------
template <uint32_t MAGIC2>
__device__ __forceinline__ void q4_pairs(const uint4 w, uint32_t (&p)[16]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
#pragma unroll
    for (int s = 0; s < 4; s++) p[4 * j + s] = ((wd[j] >> (4 * s)) & 0x000F000Fu) | MAGIC2;
  }
}

// Pairs 4g..4g+3 of a Q4 chunk, from its word g alone.
template <uint32_t MAGIC2>
__device__ __forceinline__ void q4_word_pairs(uint32_t wd, uint32_t (&p)[4]) {
#pragma unroll
  for (int s = 0; s < 4; s++) p[s] = ((wd >> (4 * s)) & 0x000F000Fu) | MAGIC2;
}

// Q3 chunk: three words W0, W1, W2. Pair i < 15 sits in word i / 5 as two
// 3-bit fields at bits 3 (i % 5) (element 2i) and 16 + 3 (i % 5) (element
// 2i + 1), so it is one shift and one and-or, like a Q4 pair; pair 15 takes
// the spare bits 15 (element 30) and 31 (element 31) of the three words, bit
// b of its codes from word b.
template <uint32_t MAGIC2>
__device__ __forceinline__ uint32_t q3_pair(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
  // i in 0..15 (compile-time after unrolling)
  if (i == 15) {
    uint32_t p = ((w0 >> 15) & 0x00010001u) | MAGIC2;
    p |= (w1 >> 14) & 0x00020002u;
    return p | ((w2 >> 13) & 0x00040004u);
  }
  const uint32_t w = (i < 5) ? w0 : (i < 10) ? w1 : w2;
  return ((w >> (3 * (i % 5))) & 0x00070007u) | MAGIC2;
}

template <uint32_t MAGIC2>
__device__ __forceinline__ void q3_pairs(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t (&p)[16]) {
#pragma unroll
  for (int i = 0; i < 16; i++) p[i] = q3_pair<MAGIC2>(w0, w1, w2, i);
}

// Pairs 4g..4g+3 of a Q3 chunk (elements 8g..8g+7).
template <uint32_t MAGIC2>
__device__ __forceinline__ void q3_group_pairs(uint32_t w0, uint32_t w1, uint32_t w2, int g, uint32_t (&p)[4]) {
#pragma unroll
  for (int s = 0; s < 4; s++) p[s] = q3_pair<MAGIC2>(w0, w1, w2, 4 * g + s);
}

static constexpr uint32_t BF16_MAGIC2 = 0x43004300u;  // bf16(128) in both halves
static constexpr uint32_t F16_MAGIC2 = 0x64006400u;   // fp16(1024) in both halves

// Offset of stored codes: stored = signed + OFF
template <int WT> struct QOff;
template <> struct QOff<MOE_W_Q4> { static constexpr int v = 8; };
template <> struct QOff<MOE_W_Q3> { static constexpr int v = 4; };

// One fp16-magic pair -> two fp32 weights scale * (code - OFF), exact:
// fma(1024 + code, s, -(1024 + OFF) * s) rounds the exact value once, and
// the exact value needs at most 15 significant bits.
__device__ __forceinline__ void f16pair_dequant(uint32_t pair, float s, float negbase,
                                                float& lo, float& hi) {
  half2_t h = __builtin_bit_cast(half2_t, pair);
  lo = __builtin_fmaf((float)h[0], s, negbase);
  hi = __builtin_fmaf((float)h[1], s, negbase);
}

// ---------------------------------------------------------------------------
// Wave reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ __forceinline__ float group_sum_f32(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace moe

namespace moe {
// ---------------------------------------------------------------------------
// DPP cross-lane helpers (no LDS traffic). Controls: quad_perm(1,0,3,2) = xor 1,
// quad_perm(2,3,0,1) = xor 2, row_half_mirror (i <-> 7-i in 8 lanes),
// row_mirror (i <-> 15-i in 16 lanes).
// ---------------------------------------------------------------------------
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
// Sum over aligned groups of 8 / 16 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8_f32(float v) {
  v += dpp_f32<DPP_XOR1>(v);
  v += dpp_f32<DPP_XOR2>(v);
  v += dpp_f32<DPP_HALF_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float sum16_f32(float v) {
  v = sum8_f32(v);
  v += dpp_f32<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ double sum16_f64(double v) {
  v += dpp_f64<DPP_XOR1>(v);
  v += dpp_f64<DPP_XOR2>(v);
  v += dpp_f64<DPP_HALF_MIRROR>(v);
  v += dpp_f64<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Whole-wave fp64 sum, fixed association ((r0 + r1) + (r2 + r3)) over 16-lane rows; uniform result.
__device__ __forceinline__ double wave_total_f64(double v) {
  v = sum16_f64(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// (value, index) ordering used by top-k: larger value first, lower index on ties.
__device__ __forceinline__ bool topk_before(double va, int ia, double vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));  // bitwise: no branches
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
  const double ov = dpp_f64<CTRL>(v);
  const int oi = dpp_i32<CTRL>(i);
  if (topk_before(ov, oi, v, i)) { v = ov; i = oi; }
}
// Wave-wide best (value, index); uniform result.
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  argmax_step<DPP_XOR1>(v, i);
  argmax_step<DPP_XOR2>(v, i);
  argmax_step<DPP_HALF_MIRROR>(v, i);
  argmax_step<DPP_MIRROR>(v, i);
  double bv = readlane_f64(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; r++) {
    const double rv = readlane_f64(v, 16 * r);
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (topk_before(rv, ri, bv, bi)) { bv = rv; bi = ri; }
  }
  v = bv;
  i = bi;
}
// Sortable 32-bit key of an fp64 value: its leading 32 bits, ordered as
// unsigned integers the way the values order.
__device__ __forceinline__ uint32_t sort_key_hi(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t k = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (uint32_t)(k >> 32);
}

// Smallest fp64 value whose sortable key has high word `hi` (low word 0).
__device__ __forceinline__ double key_floor_value(uint32_t hi) {
  const uint64_t k = (uint64_t)hi << 32;
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  const double v = __longlong_as_double((long long)b);
  return (v == v) ? v : -__builtin_inf();  // a NaN pattern (keys of -inf or below) admits every value
}

}  // namespace moe
