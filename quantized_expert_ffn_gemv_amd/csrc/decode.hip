// Decode path: batch-1 (and small-batch) MoE layer as three kernels.
//
//   A  k_dec_router_shared : router logits in fp64 (one wave per expert row)
//                            and the shared expert's gate/up GEMV + SwiGLU.
//   B  k_dec_gate_up       : ordered top-k + renormalised gates (every
//                            workgroup recomputes it from the logits), the
//                            unique-expert list of the batch, then the fused
//                            dequantise-GEMV of each selected expert's gate
//                            and up rows with the SwiGLU epilogue.
//   C  k_dec_down          : down GEMV of every selected expert and the
//                            shared expert, gate-weighted and summed per
//                            output row in a fixed order (no atomics).
//
// Weights are chunk-major (see moe.h), so the lanes of a wave that work on
// consecutive rows of one chunk read consecutive 16-byte pieces.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int DEC_THREADS = 256;

// ---------------------------------------------------------------------------
// Shared helpers
// ---------------------------------------------------------------------------

// x[t][8c .. 8c+8) as four bf16 pairs from global memory.
__device__ __forceinline__ uint4 ldg_x8(const uint16_t* x, size_t off) {
  return *reinterpret_cast<const uint4*>(x + off);
}

// Accumulate one chunk of a BF16 or F32 weight row against token activations
// held as bf16 in LDS (xs: [nt][H]).
template <int WT, int MAXB>
__device__ __forceinline__ void acc_dense_chunk(const uint8_t* wrow_chunk, const uint16_t* xs, int H,
                                                int c, int nt, float (&acc)[MAXB]) {
  if constexpr (WT == MOE_W_BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(wrow_chunk);
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < nt) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)t * H + 8 * c);
        float a = acc[t];
        a = dot2_bf16(w.x, xv.x, a);
        a = dot2_bf16(w.y, xv.y, a);
        a = dot2_bf16(w.z, xv.z, a);
        a = dot2_bf16(w.w, xv.w, a);
        acc[t] = a;
      }
    }
  } else {  // F32, chunk = 4 elements
    const float4 w = *reinterpret_cast<const float4*>(wrow_chunk);
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < nt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xs + (size_t)t * H + 4 * c);
        float a = acc[t];
        a = __builtin_fmaf(w.x, bf16_lo(xv.x), a);
        a = __builtin_fmaf(w.y, bf16_hi(xv.x), a);
        a = __builtin_fmaf(w.z, bf16_lo(xv.y), a);
        a = __builtin_fmaf(w.w, bf16_hi(xv.y), a);
        acc[t] = a;
      }
    }
  }
}

// Accumulate one 32-element quantised chunk: acc[t] += s * sum_k (code_k - OFF) x_k.
// xs: bf16 activations [nt][H] in LDS; xsum: [nt][H/32] block sums of x.
template <int WT, int MAXB>
__device__ __forceinline__ void acc_quant_chunk(const uint8_t* wchunk, float s, const uint16_t* xs,
                                                const float* xsum, int H, int c, int nt,
                                                float (&acc)[MAXB]) {
  uint32_t p[16];
  if constexpr (WT == MOE_W_Q4) {
    q4_pairs<BF16_MAGIC2>(*reinterpret_cast<const uint4*>(wchunk), p);
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(wchunk);
    q3_pairs<BF16_MAGIC2>(w[0], w[1], w[2], p);
  }
  constexpr float base = 128.0f + (float)QOff<WT>::v;
  const int nb = H >> 5;
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    if (t < nt) {
      const uint4* xv = reinterpret_cast<const uint4*>(xs + (size_t)t * H + 32 * c);
      float a = -base * xsum[t * nb + c];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint4 v = xv[q];
        a = dot2_bf16(p[4 * q + 0], v.x, a);
        a = dot2_bf16(p[4 * q + 1], v.y, a);
        a = dot2_bf16(p[4 * q + 2], v.z, a);
        a = dot2_bf16(p[4 * q + 3], v.w, a);
      }
      acc[t] = __builtin_fmaf(s, a, acc[t]);
    }
  }
}

// Stage tokens tl[0..nt) of x into LDS (bf16) and, for quantised weights,
// their 32-element block sums.
__device__ __forceinline__ void stage_x(const uint16_t* x, const int* tl, int nt, int H, uint16_t* xs,
                                        float* xsum, bool sums) {
  const int n16 = H / 8;  // 16-byte pieces per token
  for (int i = threadIdx.x; i < nt * n16; i += blockDim.x) {
    const int ti = i / n16, c = i - ti * n16;
    reinterpret_cast<uint4*>(xs + (size_t)ti * H)[c] = ldg_x8(x, (size_t)tl[ti] * H + 8 * c);
  }
  if (sums) {
    __syncthreads();
    const int nb = H >> 5;
    for (int i = threadIdx.x; i < nt * nb; i += blockDim.x) {
      const int ti = i / nb, b = i - ti * nb;
      const uint32_t* v = reinterpret_cast<const uint32_t*>(xs + (size_t)ti * H + 32 * b);
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; j++) a += bf16_lo(v[j]) + bf16_hi(v[j]);
      xsum[i] = a;
    }
  }
}

// Gate/up GEMV for NP (gate, up) row pairs of group q starting at pair j0,
// for the staged tokens. Writes h (bf16) through out(t, j) pointers.
// Thread map: rr = tid % (2*NP) (rows 0..NP-1 gate, NP..2NP-1 up),
// kpart = tid / (2*NP).
template <int WT, int MAXB, int NP>
__device__ __forceinline__ void gate_up_rows(const uint8_t* gu, const uint16_t* gus, int H, int I, int q,
                                             int j0, const uint16_t* xs, const float* xsum, int nt,
                                             float* red, float (&acc)[MAXB]) {
  constexpr int RW = 2 * NP;
  constexpr int NK = DEC_THREADS / RW;
  const int tid = threadIdx.x;
  const int rr = tid % RW, kp = tid / RW;
  const int R = 2 * I;
  const int row = 32 * q + (rr < NP ? j0 + rr : 16 + j0 + (rr - NP));
#pragma unroll
  for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
  if constexpr (WT == MOE_W_Q4 || WT == MOE_W_Q3) {
    constexpr int CB = (WT == MOE_W_Q4) ? 16 : 12;
    const int nc = H >> 5;
    for (int c = kp; c < nc; c += NK) {
      const float s = f16_to_f32(gus[(size_t)c * R + row]);
      acc_quant_chunk<WT, MAXB>(gu + ((size_t)c * R + row) * CB, s, xs, xsum, H, c, nt, acc);
    }
  } else {
    constexpr int KC = (WT == MOE_W_BF16) ? 8 : 4;
    const int nc = H / KC;
    for (int c = kp; c < nc; c += NK)
      acc_dense_chunk<WT, MAXB>(gu + ((size_t)c * R + row) * 16, xs, H, c, nt, acc);
  }
  // partials -> LDS red[kp][t][rr]
#pragma unroll
  for (int t = 0; t < MAXB; t++)
    if (t < nt) red[(kp * MAXB + t) * RW + rr] = acc[t];
  __syncthreads();
}

// Sum the K-parts for (t, j) and apply SwiGLU.
template <int MAXB, int NP>
__device__ __forceinline__ float swiglu_from_red(const float* red, int t, int j) {
  constexpr int RW = 2 * NP;
  constexpr int NK = DEC_THREADS / RW;
  float g = 0.0f, u = 0.0f;
  for (int kp = 0; kp < NK; kp++) {
    g += red[(kp * MAXB + t) * RW + j];
    u += red[(kp * MAXB + t) * RW + NP + j];
  }
  return silu_f32(g) * u;
}

// ---------------------------------------------------------------------------
// Kernel A: router logits + shared expert gate/up
// ---------------------------------------------------------------------------
template <int SWT, int MAXB, int NP>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_router_shared(LayerDev L, const uint16_t* __restrict__ x,
                                                                   int B, DecodeWs ws, int nRB) {
  const int H = L.H, E = L.E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nRB) {
    // one router row per wave, all tokens; fp32 x bf16 products are exact in fp64
    const int e = blockIdx.x * (DEC_THREADS / 64) + wave;
    if (e >= E) return;
    double acc[MAXB];
#pragma unroll
    for (int t = 0; t < MAXB; t++) acc[t] = 0.0;
    const float4* wr = reinterpret_cast<const float4*>(L.router_w + (size_t)e * H);
    const int n4 = H >> 2;
    for (int c = lane; c < n4; c += 64) {
      const float4 w = wr[c];
#pragma unroll
      for (int t = 0; t < MAXB; t++) {
        if (t < B) {
          const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)t * H + 4 * c);
          double a = acc[t];
          a = __builtin_fma((double)w.x, (double)bf16_lo(xv.x), a);
          a = __builtin_fma((double)w.y, (double)bf16_hi(xv.x), a);
          a = __builtin_fma((double)w.z, (double)bf16_lo(xv.y), a);
          a = __builtin_fma((double)w.w, (double)bf16_hi(xv.y), a);
          acc[t] = a;
        }
      }
    }
    const double b = L.router_b ? (double)L.router_b[e] : 0.0;
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < B) {
        const double v = wave_sum_f64(acc[t]);
        if (lane == 0) ws.logits[(size_t)t * E + e] = v + b;
      }
    }
    return;
  }
  // shared expert gate/up for NP pairs
  extern __shared__ __align__(16) uint8_t smem[];
  const int I = L.I;
  const int bpq = 16 / NP;
  const int b = blockIdx.x - nRB;
  const int q = b / bpq, j0 = (b % bpq) * NP;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)B * H * 2);
  int tl[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) tl[t] = t;
  stage_x(x, tl, B, H, xs, nullptr, false);
  __syncthreads();
  float acc[MAXB];
  gate_up_rows<SWT, MAXB, NP>(L.sgu, nullptr, H, I, q, j0, xs, nullptr, B, red, acc);
  for (int i = threadIdx.x; i < B * NP; i += DEC_THREADS) {
    const int t = i / NP, j = i - t * NP;
    const float hv = swiglu_from_red<MAXB, NP>(red, t, j);
    ws.hs[(size_t)t * I + 16 * q + j0 + j] = f32_to_bf16(hv);
  }
}

// ---------------------------------------------------------------------------
// Routing inside a workgroup: ordered top-k + gates for tokens 0..B-1,
// results in LDS (s_idx [B][k], s_gate [B][k]).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const double* __restrict__ logits, int E, int k, int lane,
                                          int* s_idx, float* s_gate) {
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? logits[e] : -__builtin_inf();
  }
  double m = 0.0, myv = -__builtin_inf();
  int myi = 0;
  for (int r = 0; r < k; r++) {
    double best = -__builtin_inf();
    int bi = 0x7FFFFFFF;
    // within a lane, experts lane + 64 i rise with i: strict > keeps the lower index on ties
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int e = lane + 64 * i;
      if (e < E && v[i] > best) { best = v[i]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (lane + 64 * i == bi) v[i] = -__builtin_inf();
    if (r == 0) m = best;
    if (lane == r) { myv = best; myi = bi; }
  }
  // gates: softmax over the selected logits (equal to the renormalised softmax over all E)
  const double ev = (lane < k) ? exp(myv - m) : 0.0;
  const double z = wave_sum_f64(ev);
  if (lane < k) {
    s_idx[lane] = myi;
    s_gate[lane] = (float)(ev / z);
  }
}

// ---------------------------------------------------------------------------
// Kernel B: routing + routed gate/up
// ---------------------------------------------------------------------------
template <int WT, int MAXB, int NP>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_gate_up(LayerDev L, const uint16_t* __restrict__ x, int B,
                                                             DecodeWs ws, int32_t* idx_out, float* gate_out) {
  const int H = L.H, I = L.I, E = L.E, k = L.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int s_idx[MAXB * 16];
  __shared__ float s_gate[MAXB * 16];
  __shared__ int s_uniq[MAXB * 16];
  __shared__ uint32_t s_mask[MAXB * 16];
  __shared__ int s_nu;
  __shared__ int s_tl[MAXB];
  extern __shared__ __align__(16) uint8_t smem[];

  for (int t = wave; t < B; t += DEC_THREADS / 64)
    wave_topk(ws.logits + (size_t)t * E, E, k, lane, s_idx + t * k, s_gate + t * k);
  __syncthreads();
  const int nslot = B * k;
  if (MAXB == 1) {
    if (threadIdx.x < k) { s_uniq[threadIdx.x] = s_idx[threadIdx.x]; s_mask[threadIdx.x] = 1u; }
    if (threadIdx.x == 0) s_nu = k;
    __syncthreads();
  } else {
    // unique experts in first-occurrence (slot) order, with the tokens using each
    int* mark = reinterpret_cast<int*>(smem);  // [E], reuses the dynamic LDS before staging
    for (int e = threadIdx.x; e < E; e += DEC_THREADS) mark[e] = 0x7FFFFFFF;
    __syncthreads();
    if ((int)threadIdx.x < nslot) atomicMin(&mark[s_idx[threadIdx.x]], (int)threadIdx.x);
    __syncthreads();
    // first occurrences, ranked by slot order (nslot <= 256 = one pass)
    const bool first = (int)threadIdx.x < nslot && mark[s_idx[threadIdx.x]] == (int)threadIdx.x;
    __shared__ int s_wcnt[DEC_THREADS / 64];
    __shared__ int s_uid[MAXB * 16];
    const uint64_t bal = __ballot(first);
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; w++) base += s_wcnt[w];
    const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
    if (first) { s_uniq[rank] = s_idx[threadIdx.x]; s_mask[rank] = 0u; s_uid[threadIdx.x] = rank; }
    if (threadIdx.x == 0) {
      int n = 0;
      for (int w = 0; w < DEC_THREADS / 64; w++) n += s_wcnt[w];
      s_nu = n;
    }
    __syncthreads();
    if ((int)threadIdx.x < nslot) {
      const int u = s_uid[mark[s_idx[threadIdx.x]]];
      atomicOr(&s_mask[u], 1u << (threadIdx.x / k));
    }
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < nslot; i += DEC_THREADS) {
      ws.idx[i] = s_idx[i];
      ws.gates[i] = s_gate[i];
      if (idx_out) idx_out[i] = s_idx[i];
      if (gate_out) gate_out[i] = s_gate[i];
    }
    for (int i = threadIdx.x; i < s_nu; i += DEC_THREADS) {
      ws.uniq[1 + i] = s_uniq[i];
      ws.tokmask[i] = s_mask[i];
    }
    if (threadIdx.x == 0) ws.uniq[0] = s_nu;
  }
  // this workgroup's (unique expert, row pairs)
  const int bpq = 16 / NP;
  const int gpe = (I / 16) * bpq;  // workgroups per expert
  const int u = blockIdx.x / gpe;
  if (u >= s_nu) return;
  const int r = blockIdx.x - u * gpe;
  const int q = r / bpq, j0 = (r % bpq) * NP;
  const int e = s_uniq[u];
  const uint32_t mask = s_mask[u];
  if (threadIdx.x == 0) {
    int n = 0;
    for (int t = 0; t < B; t++)
      if (mask & (1u << t)) s_tl[n++] = t;
  }
  __syncthreads();
  const int nt = __popc(mask);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)nt * H * 2);
  float* red = xsum + (size_t)nt * (H >> 5);
  constexpr bool quant = (WT == MOE_W_Q4 || WT == MOE_W_Q3);
  stage_x(x, s_tl, nt, H, xs, xsum, quant);
  __syncthreads();
  float acc[MAXB];
  gate_up_rows<WT, MAXB, NP>(L.gu + (size_t)e * L.gu_stride, quant ? L.gu_s + (size_t)e * L.gu_s_stride : nullptr,
                             H, I, q, j0, xs, xsum, nt, red, acc);
  // SwiGLU, bf16 h, and the sum of this workgroup's NP bf16 h values per token
  float* hv_lds = red + (DEC_THREADS / (2 * NP)) * MAXB * 2 * NP;  // [nt][NP]
  __syncthreads();
  for (int i = threadIdx.x; i < nt * NP; i += DEC_THREADS) {
    const int ti = i / NP, j = i - ti * NP;
    const int t = s_tl[ti];
    int slot = 0;
    for (int jj = 0; jj < k; jj++)
      if (s_idx[t * k + jj] == e) slot = jj;
    const uint16_t hb = f32_to_bf16(swiglu_from_red<MAXB, NP>(red, ti, j));
    ws.h[((size_t)t * k + slot) * I + 16 * q + j0 + j] = hb;
    hv_lds[ti * NP + j] = bf16_to_f32(hb);
  }
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int ti = threadIdx.x, t = s_tl[ti];
    int slot = 0;
    for (int jj = 0; jj < k; jj++)
      if (s_idx[t * k + jj] == e) slot = jj;
    float a = 0.0f;
    for (int j = 0; j < NP; j++) a += hv_lds[ti * NP + j];
    ws.hpart[((size_t)t * k + slot) * (I / NP) + (16 * q + j0) / NP] = a;
  }
}

// ---------------------------------------------------------------------------
// Kernel C: down GEMV of selected + shared experts, gated sum per row
// ---------------------------------------------------------------------------
constexpr int DC_ROWS = 8;
constexpr int DC_THREADS = 128;
constexpr int DC_KP = DC_THREADS / DC_ROWS;  // 16 K-parts

// One down chunk of expert weights against one h row (bf16 pairs in hrow):
// returns sum over the chunk of w * h (scale applied for quantised weights).
template <int WT>
__device__ __forceinline__ float down_chunk(const uint8_t* dn, const uint16_t* dns, int H, int row, int c,
                                            const uint16_t* hrow, float hsum_c) {
  if constexpr (WT == MOE_W_Q4 || WT == MOE_W_Q3) {
    constexpr int CB = (WT == MOE_W_Q4) ? 16 : 12;
    uint32_t p[16];
    if constexpr (WT == MOE_W_Q4) {
      q4_pairs<BF16_MAGIC2>(*reinterpret_cast<const uint4*>(dn + ((size_t)c * H + row) * CB), p);
    } else {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(dn + ((size_t)c * H + row) * CB);
      q3_pairs<BF16_MAGIC2>(w[0], w[1], w[2], p);
    }
    constexpr float base = 128.0f + (float)QOff<WT>::v;
    const uint4* hv = reinterpret_cast<const uint4*>(hrow + 32 * c);
    float a = -base * hsum_c;
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      const uint4 v = hv[qq];
      a = dot2_bf16(p[4 * qq + 0], v.x, a);
      a = dot2_bf16(p[4 * qq + 1], v.y, a);
      a = dot2_bf16(p[4 * qq + 2], v.z, a);
      a = dot2_bf16(p[4 * qq + 3], v.w, a);
    }
    return f16_to_f32(dns[(size_t)c * H + row]) * a;
  } else {
    float one[1] = {0.0f};
    acc_dense_chunk<WT, 1>(dn + ((size_t)c * H + row) * 16, hrow, 0, c, 1, one);
    return one[0];
  }
}

template <int WT, int SWT, int MAXB>
__global__ __launch_bounds__(DC_THREADS) void k_dec_down(LayerDev L, int B, DecodeWs ws, uint16_t* __restrict__ y,
                                                         int stage_lds) {
  const int H = L.H, I = L.I, k = L.k;
  const int tid = threadIdx.x;
  const int rr = tid % DC_ROWS, kp = tid / DC_ROWS;
  const int row = blockIdx.x * DC_ROWS + rr;
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool quant = (WT == MOE_W_Q4 || WT == MOE_W_Q3);
  const int nslot = B * k;
  const bool has_shared = (SWT != MOE_W_NONE);
  const int nrow = nslot + (has_shared ? B : 0);
  const int nb = I >> 5;
  const int hp = I / DEC_NP;  // h partial sums per slot
  // LDS: red [MAXB][KP][ROWS] f32 | slot-of(u,t) [MAXB*16] | hsum [nslot][nb] | (staged h)
  float* red = reinterpret_cast<float*>(smem);
  int* s_slot = reinterpret_cast<int*>(red + MAXB * DC_KP * DC_ROWS);
  float* hsum = reinterpret_cast<float*>(s_slot + MAXB * 16);
  uint16_t* hst = reinterpret_cast<uint16_t*>(hsum + nslot * nb);
  if (stage_lds) {
    const int n16 = I / 8;
    for (int i = tid; i < nrow * n16; i += DC_THREADS) {
      const int s = i / n16, c = i - s * n16;
      const uint16_t* src = (s < nslot) ? ws.h + (size_t)s * I : ws.hs + (size_t)(s - nslot) * I;
      reinterpret_cast<uint4*>(hst + (size_t)s * I)[c] = reinterpret_cast<const uint4*>(src)[c];
    }
  }
  if (quant) {
    for (int i = tid; i < nslot * nb; i += DC_THREADS) {
      const int s = i / nb, c = i - s * nb;
      const float* hpp = ws.hpart + (size_t)s * hp + c * (32 / DEC_NP);
      float a = 0.0f;
      for (int j = 0; j < 32 / DEC_NP; j++) a += hpp[j];
      hsum[i] = a;
    }
  }
  const int nu = ws.uniq[0];
  // slot index of (unique expert u, token t): s_slot[u*MAXB + t] = t*k + j
  for (int i = tid; i < nu * B; i += DC_THREADS) {
    const int u = i / B, t = i - u * B;
    const int e = ws.uniq[1 + u];
    int slot = -1;
    for (int j = 0; j < k; j++)
      if (ws.idx[t * k + j] == e) slot = t * k + j;
    if (u < 16) s_slot[u * MAXB + t] = slot;
  }
  __syncthreads();
  float acc[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
  const uint16_t* hbase = stage_lds ? hst : ws.h;
  if (row < H) {
    for (int u = 0; u < nu; u++) {
      const int e = ws.uniq[1 + u];
      const uint8_t* dn = L.dn + (size_t)e * L.dn_stride;
      const uint16_t* dns = quant ? L.dn_s + (size_t)e * L.dn_s_stride : nullptr;
      constexpr int KC = quant ? 32 : (WT == MOE_W_BF16 ? 8 : 4);
      const int nc = I / KC;
#pragma unroll
      for (int t = 0; t < MAXB; t++) {
        if (t < B) {
          int sr;
          if (MAXB == 1) {
            sr = u;
          } else if (u < 16) {
            sr = s_slot[u * MAXB + t];
          } else {
            sr = -1;
            for (int j = 0; j < k; j++)
              if (ws.idx[t * k + j] == e) sr = t * k + j;
          }
          if (sr >= 0) {
            const float g = ws.gates[sr];
            const uint16_t* hrow = hbase + (size_t)sr * I;
            float a = 0.0f;
            for (int c = kp; c < nc; c += DC_KP)
              a += down_chunk<WT>(dn, dns, H, row, c, hrow, quant ? hsum[sr * nb + (c * KC >> 5)] : 0.0f);
            acc[t] = __builtin_fmaf(g, a, acc[t]);
          }
        }
      }
    }
    if (has_shared) {
      constexpr int SKC = (SWT == MOE_W_BF16) ? 8 : 4;
      const int nc = I / SKC;
      const uint16_t* hsb = stage_lds ? hst + (size_t)nslot * I : ws.hs;
      for (int c = kp; c < nc; c += DC_KP) acc_dense_chunk<SWT, MAXB>(L.sdn + ((size_t)c * H + row) * 16, hsb, I, c, B, acc);
    }
  }
  // reduce over the 16 K-parts: lanes rr + 8*kp; kp spans both waves
#pragma unroll
  for (int t = 0; t < MAXB; t++)
    if (t < B) red[(t * DC_KP + kp) * DC_ROWS + rr] = acc[t];
  __syncthreads();
  for (int i = tid; i < B * DC_ROWS; i += DC_THREADS) {
    const int t = i / DC_ROWS, r2 = i - t * DC_ROWS;
    const int orow = blockIdx.x * DC_ROWS + r2;
    float sum = 0.0f;
    for (int p = 0; p < DC_KP; p++) sum += red[(t * DC_KP + p) * DC_ROWS + r2];
    if (orow < H) y[(size_t)t * H + orow] = f32_to_bf16(sum);
  }
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
template <int WT, int SWT, int MAXB>
static hipError_t launch_decode_t(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out,
                                  float* gate_out, const DecodeWs& ws, hipStream_t st) {
  constexpr int NP = DEC_NP;
  const int H = L.H, I = L.I, E = L.E, k = L.k;
  // A
  const int nRB = (E + 3) / 4;
  const int nSB = (SWT != MOE_W_NONE) ? (I / 16) * (16 / NP) : 0;
  {
    constexpr int SW = (SWT == MOE_W_NONE) ? MOE_W_BF16 : SWT;
    const size_t lds = (size_t)B * H * 2 + (size_t)(DEC_THREADS / (2 * NP)) * MAXB * 2 * NP * 4;
    timer_begin(KC_DEC_ROUTER_SHARED, st);
    hipLaunchKernelGGL((k_dec_router_shared<SW, MAXB, NP>), dim3(nRB + nSB), dim3(DEC_THREADS), lds, st, L, x, B,
                       ws, nRB);
    timer_end(KC_DEC_ROUTER_SHARED, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // B
  {
    const int maxU = (B * k < E) ? B * k : E;
    const int gpe = (I / 16) * (16 / NP);
    const size_t stage = (size_t)B * H * 2 + (size_t)B * (H / 32) * 4 +
                         (size_t)(DEC_THREADS / (2 * NP)) * MAXB * 2 * NP * 4 + (size_t)MAXB * NP * 4;
    const size_t lds = (stage > (size_t)E * 4) ? stage : (size_t)E * 4;
    timer_begin(KC_DEC_GATE_UP, st);
    hipLaunchKernelGGL((k_dec_gate_up<WT, MAXB, NP>), dim3(maxU * gpe), dim3(DEC_THREADS), lds, st, L, x, B, ws,
                       idx_out, gate_out);
    timer_end(KC_DEC_GATE_UP, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // C
  {
    const int nslot = B * k;
    const int nrow = nslot + (SWT != MOE_W_NONE ? B : 0);
    const size_t fixed = (size_t)MAXB * DC_KP * DC_ROWS * 4 + (size_t)MAXB * 16 * 4 + (size_t)nslot * (I / 32) * 4;
    const size_t hbytes = (size_t)nrow * I * 2;
    const int stage = (fixed + hbytes <= 48 * 1024) ? 1 : 0;
    const size_t lds = fixed + (stage ? hbytes : 0);
    timer_begin(KC_DEC_DOWN, st);
    hipLaunchKernelGGL((k_dec_down<WT, SWT, MAXB>), dim3((H + DC_ROWS - 1) / DC_ROWS), dim3(DC_THREADS), lds, st,
                       L, B, ws, y, stage);
    timer_end(KC_DEC_DOWN, st);
    return hipGetLastError();
  }
}

template <int WT, int SWT>
static hipError_t launch_decode_b(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                                  const DecodeWs& ws, hipStream_t st) {
  if (B == 1) return launch_decode_t<WT, SWT, 1>(L, x, B, y, io, go, ws, st);
  return launch_decode_t<WT, SWT, 16>(L, x, B, y, io, go, ws, st);
}

template <int WT>
static hipError_t launch_decode_s(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                                  const DecodeWs& ws, hipStream_t st) {
  switch (L.swt) {
    case MOE_W_BF16: return launch_decode_b<WT, MOE_W_BF16>(L, x, B, y, io, go, ws, st);
    case MOE_W_F32: return launch_decode_b<WT, MOE_W_F32>(L, x, B, y, io, go, ws, st);
    default: return launch_decode_b<WT, MOE_W_NONE>(L, x, B, y, io, go, ws, st);
  }
}

hipError_t launch_decode(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out, float* gate_out,
                         const DecodeWs& ws, hipStream_t st) {
  switch (L.wt) {
    case MOE_W_Q4: return launch_decode_s<MOE_W_Q4>(L, x, B, y, idx_out, gate_out, ws, st);
    case MOE_W_Q3: return launch_decode_s<MOE_W_Q3>(L, x, B, y, idx_out, gate_out, ws, st);
    case MOE_W_BF16: return launch_decode_s<MOE_W_BF16>(L, x, B, y, idx_out, gate_out, ws, st);
    default: return launch_decode_s<MOE_W_F32>(L, x, B, y, idx_out, gate_out, ws, st);
  }
}

}  // namespace moe
