// Device helpers of the decode kernels: weight chunks, dot products against
// LDS-staged bf16 vectors, and the ordered top-k of one token's logits.
#pragma once
#include "moe_device.h"

namespace moe {

template <int WT> constexpr int kchunk() { return WT == MOE_W_F32 ? 4 : (WT == MOE_W_BF16 ? 8 : 32); }
template <int WT> constexpr bool is_q() { return WT == MOE_W_Q4 || WT == MOE_W_Q3; }

struct Raw {
  uint32_t w[4];
};

template <int WT>
__device__ __forceinline__ Raw load_chunk(const uint8_t* base, size_t ci) {
  Raw r;
  if constexpr (WT == MOE_W_Q3) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(base + ci * 12);
    r.w[0] = p[0];
    r.w[1] = p[1];
    r.w[2] = p[2];
    r.w[3] = 0;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(base + ci * 16);
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
    r.w[3] = v.w;
  }
  return r;
}

// sum_k (code_k - OFF) * a_k over a 32-element chunk (`a`: 32 bf16 values in
// LDS, asum their sum), in two parts: qunpack32 turns the chunk into 16 bf16
// pairs (128 + code each, exact), qdot32_p dots them with the activations in
// four independent dot2 chains (so a chunk used by several tokens is
// unpacked once); qdot32 does both. The caller scales.
template <int WT>
__device__ __forceinline__ void qunpack32(const Raw& r, uint32_t (&p)[16]) {
  if constexpr (WT == MOE_W_Q4) {
    q4_pairs<BF16_MAGIC2>(make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]), p);
  } else {
    q3_pairs<BF16_MAGIC2>(r.w[0], r.w[1], r.w[2], p);
  }
}
template <int WT>
__device__ __forceinline__ float qdot32_p(const uint32_t (&p)[16], const uint16_t* a, float asum) {
  const uint4* av = reinterpret_cast<const uint4*>(a);
  float c0 = -(128.0f + (float)QOff<WT>::v) * asum, c1 = 0.0f, c2 = 0.0f, c3 = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint4 v = av[q];
    c0 = dot2_bf16(p[4 * q + 0], v.x, c0);
    c1 = dot2_bf16(p[4 * q + 1], v.y, c1);
    c2 = dot2_bf16(p[4 * q + 2], v.z, c2);
    c3 = dot2_bf16(p[4 * q + 3], v.w, c3);
  }
  return (c0 + c1) + (c2 + c3);
}
template <int WT>
__device__ __forceinline__ float qdot32(const Raw& r, const uint16_t* a, float asum) {
  uint32_t p[16];
  qunpack32<WT>(r, p);
  return qdot32_p<WT>(p, a, asum);
}

// Dot of one dense chunk (8 bf16 or 4 fp32 weights) with bf16 activations.
template <int WT>
__device__ __forceinline__ float ddot(const Raw& r, const uint16_t* a, float acc) {
  if constexpr (WT == MOE_W_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(a);
    float c1 = 0.0f;
    acc = dot2_bf16(r.w[0], v.x, acc);
    c1 = dot2_bf16(r.w[1], v.y, c1);
    acc = dot2_bf16(r.w[2], v.z, acc);
    c1 = dot2_bf16(r.w[3], v.w, c1);
    return acc + c1;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(a);
    acc = __builtin_fmaf(__uint_as_float(r.w[0]), bf16_lo(v.x), acc);
    acc = __builtin_fmaf(__uint_as_float(r.w[1]), bf16_hi(v.x), acc);
    acc = __builtin_fmaf(__uint_as_float(r.w[2]), bf16_lo(v.y), acc);
    acc = __builtin_fmaf(__uint_as_float(r.w[3]), bf16_hi(v.y), acc);
    return acc;
  }
}

// Copy B tokens of x into LDS (bf16) and, if asked, their 32-element block sums.
template <int NT>
__device__ __forceinline__ void stage_tokens(const uint16_t* __restrict__ x, int B, int H, uint16_t* xs, float* xsum) {
  const int n16 = H / 8;
  for (int i = threadIdx.x; i < B * n16; i += NT) reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
  if (xsum) {
    __syncthreads();
    const int nb = H >> 5;
    for (int i = threadIdx.x; i < B * nb; i += NT) {
      const uint32_t* v = reinterpret_cast<const uint32_t*>(xs + (size_t)i * 32);
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; j++) a += bf16_lo(v[j]) + bf16_hi(v[j]);
      xsum[i] = a;
    }
  }
}

__device__ __forceinline__ float wave_total_f32(float v) {
  v = sum16_f32(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// ---------------------------------------------------------------------------
// Ordered top-k of one token's logits in one wave (lane holds the logits of
// experts lane + 64 i, i < NV, so E <= 64 NV; invalid entries are -inf).
//   1. each lane's best value; its 32-bit sortable key (sign, exponent and
//      leading mantissa bits of the fp64 logit) with the low 6 bits replaced
//      by 63 - lane, so the 64 keys are distinct and never contradict value
//      order at the 26 bits they keep;
//   2. the larger key of each lane pair (32 keys); rank of every pair key
//      by counting (keys exchanged through LDS); tau = the key of rank k-1,
//      and tv = the smallest fp64 value whose key truncates to tau's. Any
//      value below tv is beaten by the bests of k pairs, so it cannot be in
//      the top-k;
//   3. candidates = values >= tv, compacted to LDS (candidate lanes write);
//   4. exact rank of each candidate among the candidates (fp64 value, then
//      index): four lanes per candidate up to 16 candidates (the usual
//      case), else one lane each, the others broadcast through scalar
//      registers; picks and orders the k winners.
// Only massively tied logits (more than TOPK_CMAX candidates) take the slow
// path: k rounds of a wave arg-max. Order: larger logit first, lower expert
// index on ties. Lane r < k ends with expert r and its renormalised gate,
// the softmax of the k selected logits (equal to p_S / sum of p over S):
// exp in fp32 of the fp64 difference to the largest, summed in fp64.
// ---------------------------------------------------------------------------
constexpr int TOPK_CMAX = 128;
// bytes per wave: 64 keys, (TOPK_CMAX + 64) candidate slots, 16 outputs; slots are 16 B (value, index)
constexpr size_t TOPK_SCRATCH = 64 * 4 + (size_t)(TOPK_CMAX + 64) * 16 + 16 * 16;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct TopkSlot {  // 16 bytes in LDS
  double v;
  int i;
  int pad;
};

// Gates of the k ordered winners S_o[0 .. k) (k <= 16: lanes 0..15, one
// DPP row): lane r < k ends with expert r and the softmax of the k selected
// logits, exp in fp32 of the fp64 difference to the largest, summed in fp64.
__device__ __forceinline__ void topk_gates(const TopkSlot* S_o, int E, int k, int lane, int& my_idx, float& my_gate) {
  const TopkSlot o = S_o[lane < k ? lane : 0];
  const double mv = S_o[0].v;
  const float ef = (lane < k) ? expf((float)(o.v - mv)) : 0.0f;
  const double z = sum16_f64((double)ef);
  int ix = (lane < k) ? o.i : 0;
  ix = ix < 0 ? 0 : (ix >= E ? E - 1 : ix);  // in range whatever the logits held
  my_idx = ix;
  my_gate = (lane < k) ? (float)((double)ef / z) : 0.0f;
}

// The k ordered winners to S_o[0 .. k) (LDS; visible to the wave after
// wave_lds_sync).
template <int NV>
__device__ __forceinline__ void wave_topk_order(const double (&v)[NV], int E, int k, int lane, uint8_t* scratch,
                                                TopkSlot* S_o) {
  uint32_t* S_key = reinterpret_cast<uint32_t*>(scratch);
  TopkSlot* S_c = reinterpret_cast<TopkSlot*>(scratch + 256);  // [TOPK_CMAX] candidates + [64] per-lane scratch
  const int nv = (E + 63) >> 6;  // value slots in use (uniform)
  // 1. lane best and its distinct key
  double bv = -__builtin_inf();
#pragma unroll
  for (int i = 0; i < NV; i++)
    if (i < nv) bv = (v[i] > bv) ? v[i] : bv;
  const uint32_t key = (sort_key_hi(bv) & ~63u) | (uint32_t)(63 - lane);
  // the larger key of each lane pair: 32 distinct keys, each the maximum of
  // 2 NV values (k <= 16 <= 32)
  const uint32_t pk = max(key, (uint32_t)dpp_i32<DPP_XOR1>((int)key));
  if ((lane & 1) == 0) S_key[lane >> 1] = pk;
  wave_lds_sync();
  // 2. rank of pair (lane & 31)'s key among the 32 (lanes < 32), and the
  //    threshold: the k-th largest pair key; k pairs hold a value >= it, so
  //    every top-k value is >= it (half the compares of ranking 64 lane keys)
  const uint32_t mine = S_key[lane & 31];
  int r0 = 0, r1 = 0;
  const uint4* kv = reinterpret_cast<const uint4*>(S_key);
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint4 q = kv[j], q2 = kv[j + 1];
    r0 += (int)(q.x > mine) + (int)(q.y > mine) + (int)(q.z > mine) + (int)(q.w > mine);
    r1 += (int)(q2.x > mine) + (int)(q2.y > mine) + (int)(q2.z > mine) + (int)(q2.w > mine);
  }
  const uint64_t sel = __ballot((lane < 32) & (r0 + r1 == k - 1));
  const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)mine, __ffsll((long long)sel) - 1) & ~63u;
  const double tv = key_floor_value(tau);
  // 3. candidates, compacted in (slot, lane) order
  int base = 0;
#pragma unroll
  for (int i = 0; i < NV; i++) {
    if (i < nv) {
      const int e = lane + 64 * i;
      const bool cand = (e < E) & (v[i] >= tv);
      const uint64_t bal = __ballot(cand);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      // every lane writes (no branch): non-candidates to their own slot past
      // the candidate area
      const int wp = (cand & (pos < TOPK_CMAX)) ? pos : TOPK_CMAX + lane;
      S_c[wp].v = v[i];
      S_c[wp].i = e;
      base += __popcll(bal);
    }
  }
  const int nc = base;
  wave_lds_sync();
  if (nc <= 16) {
    // 4'. the usual case (about 11 candidates): four lanes per candidate,
    //     each comparing it with every fourth candidate (broadcast LDS
    //     reads), the four counts summed across the quad; a loop of scalar
    //     broadcasts over the candidates costs ~3x as much
    const int c = lane >> 2, g = lane & 3;
    const TopkSlot me = S_c[c < nc ? c : 0];
    int rk = 0;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int j = g + 4 * jj;
      const TopkSlot o = S_c[j < nc ? j : 0];
      rk += (int)((j < nc) & topk_before(o.v, o.i, me.v, me.i));
    }
    rk += dpp_i32<DPP_XOR1>(rk);
    rk += dpp_i32<DPP_XOR2>(rk);
    if ((g == 0) & (c < nc) & (rk < k)) {
      S_o[rk].v = me.v;
      S_o[rk].i = me.i;
    }
  } else if (nc <= 64) {
    // 4. exact ranks: candidate c sits in lane c; each candidate in turn is
    //    broadcast through scalar registers and every lane compares
    const double cvv = (lane < nc) ? S_c[lane < nc ? lane : 0].v : -__builtin_inf();
    const int cii = (lane < nc) ? S_c[lane < nc ? lane : 0].i : 0x7FFFFFFF;
    int rk = 0;
    for (int j = 0; j < nc; j++) {
      const double sv = readlane_f64(cvv, j);
      const int si = __builtin_amdgcn_readlane(cii, j);
      rk += topk_before(sv, si, cvv, cii);
    }
    if (lane < nc && rk < k) {
      S_o[rk].v = cvv;
      S_o[rk].i = cii;
    }
  } else if (nc <= TOPK_CMAX) {
    // 4'. many candidates: each lane ranks several
    for (int c = lane; c < nc; c += 64) {
      const double cvv = S_c[c].v;
      const int cii = S_c[c].i;
      int q0 = 0;
      for (int j = 0; j < nc; j++) q0 += topk_before(S_c[j].v, S_c[j].i, cvv, cii);
      if (q0 < k) {
        S_o[q0].v = cvv;
        S_o[q0].i = cii;
      }
    }
  } else {
    // massively tied keys: k rounds of a wave arg-max over all values
    double w[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) w[i] = v[i];
    for (int r = 0; r < k; r++) {
      double best = -__builtin_inf();
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < NV; i++) {
        const int e = lane + 64 * i;
        const bool take = (e < E) & (w[i] > best);
        best = take ? w[i] : best;
        bi = take ? e : bi;
      }
      wave_argmax(best, bi);
#pragma unroll
      for (int i = 0; i < NV; i++)
        if (lane + 64 * i == bi) w[i] = -__builtin_inf();
      if (lane == 0) {
        S_o[r].v = best;
        S_o[r].i = bi;
      }
    }
  }
}

template <int NV>
__device__ __forceinline__ void wave_topk(const double (&v)[NV], int E, int k, int lane, uint8_t* scratch, int& my_idx,
                                          float& my_gate) {
  TopkSlot* S_o = reinterpret_cast<TopkSlot*>(scratch + 256) + TOPK_CMAX + 64;  // [16] ordered winners
  wave_topk_order(v, E, k, lane, scratch, S_o);
  wave_lds_sync();
  topk_gates(S_o, E, k, lane, my_idx, my_gate);
}

}  // namespace moe
