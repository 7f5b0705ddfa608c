// Decode path: one MoE layer for B <= 8 tokens as four kernels. (Batch 1
// takes the one-kernel path of decode1.hip whenever its shape fits there.)
//
//   A  k_dec_a     : router logits in fp64 (one wave per expert row; an fp32
//                    weight times a bf16 activation is exact in fp64), and
//                    the whole shared expert: each workgroup owns 8
//                    intermediate columns, computes them (gate/up GEMV +
//                    SwiGLU) and their contribution to every output row (a
//                    partial down product).
//   R  k_dec_route : one workgroup: ordered top-k and renormalised gates of
//                    every token, the batch's unique-expert list and, per
//                    unique expert, the mask of the tokens that chose it.
//   B  k_dec_b     : per (unique expert, G intermediate columns; G = 32 for
//                    quantised weights, 16 for dense): fused
//                    dequantise-GEMV of the 2G gate/up rows for the tokens
//                    in the expert's mask, SwiGLU, and the gated partial down
//                    product over those G columns. The down weights are
//                    loaded together with the gate/up weights, so the down
//                    projection adds no memory round trip.
//   C  k_dec_c     : y = sum of the partial products, in a fixed order.
//
// No float atomics: every partial lands in its own fp32 slot and the sum
// order is fixed, so results are bitwise reproducible. Threads issue all
// of their weight loads before computing; lane partial sums reduce by DPP.
#include "moe_device.h"
#include "moe_internal.h"
#include "dec_common.h"

namespace moe {

constexpr int DA_THREADS = 512;  // kernel A: 8 waves
constexpr int DB_THREADS = 512;  // kernel B: 8 waves
constexpr int DC_THREADS = 256;  // kernel C
constexpr int DC_ROWS = 32;      // output rows per kernel-C workgroup (128-byte row segments per partial)
constexpr int DC_SPLIT = DC_THREADS / DC_ROWS;

// ---------------------------------------------------------------------------
// Down-projection pieces: NCOL consecutive intermediate columns (16 for a
// routed workgroup over dense weights, 8 for a shared-expert workgroup) of
// one output row of a chunk-major D[H][I], and their dot with NCOL bf16 h
// values (NCOL/2 pairs). Quantised routed workgroups take whole chunks.
// ---------------------------------------------------------------------------
template <int WT, int NCOL>
struct DownPiece {
  static constexpr int NW = is_q<WT>() ? 2 : (WT == MOE_W_F32 ? NCOL : NCOL / 2);
  uint32_t w[NW];
  float s;
};

template <int WT, int NCOL>
__device__ __forceinline__ void load_down_piece(const uint8_t* dn, const uint16_t* dns, int H, int row, int col0,
                                                DownPiece<WT, NCOL>& d) {
  if constexpr (is_q<WT>()) {
    static_assert(NCOL == 16, "quantised down pieces are half chunks");
    const int c = col0 >> 5, half = (col0 >> 4) & 1;
    const uint8_t* base = dn + ((size_t)c * H + row) * (WT == MOE_W_Q4 ? 16 : 12);
    if constexpr (WT == MOE_W_Q4) {
      const uint2 v = *reinterpret_cast<const uint2*>(base + 8 * half);  // words 2h, 2h+1
      d.w[0] = v.x;
      d.w[1] = v.y;
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(base);
      d.w[0] = p[half];  // L0 or L1
      d.w[1] = p[2];     // HB
    }
    d.s = f16_to_f32(dns[(size_t)c * H + row]);
  } else {
    constexpr int KC = kchunk<WT>();
    constexpr int ES = (WT == MOE_W_F32) ? 4 : 2;
    if constexpr (NCOL >= KC) {
      constexpr int NCH = NCOL / KC;
#pragma unroll
      for (int i = 0; i < NCH; i++) {
        const uint4 v = *reinterpret_cast<const uint4*>(dn + ((size_t)(col0 / KC + i) * H + row) * 16);
        d.w[4 * i] = v.x;
        d.w[4 * i + 1] = v.y;
        d.w[4 * i + 2] = v.z;
        d.w[4 * i + 3] = v.w;
      }
    } else {  // part of one chunk: NCOL * ES bytes (8 for 4 bf16 columns)
      static_assert(NCOL * ES == 8, "sub-chunk pieces are 8 bytes");
      const uint2 v = *reinterpret_cast<const uint2*>(dn + ((size_t)(col0 / KC) * H + row) * 16 + (col0 % KC) * ES);
      d.w[0] = v.x;
      d.w[1] = v.y;
    }
    d.s = 1.0f;
  }
}

// the 8 code pairs of a quantised piece as bf16 (128 + code), once per piece
template <int WT, int NCOL>
__device__ __forceinline__ void down_piece_unpack(const DownPiece<WT, NCOL>& d, int half, uint32_t (&p)[8]) {
  if constexpr (is_q<WT>()) {
    if constexpr (WT == MOE_W_Q4) {
#pragma unroll
      for (int w = 0; w < 2; w++)
#pragma unroll
        for (int s = 0; s < 4; s++) p[4 * w + s] = ((d.w[w] >> (4 * s)) & 0x000F000Fu) | BF16_MAGIC2;
    } else {
      const uint32_t hsh = d.w[1] >> (8 * half);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t v = ((d.w[0] >> (2 * i)) & 0x00030003u) | BF16_MAGIC2;
        const uint32_t h = (i >= 2) ? (hsh >> (i - 2)) : (hsh << (2 - i));
        p[i] = v | (h & 0x00040004u);
      }
    }
  }
}
// its dot with one token's 16 bf16 h values (hp, 8 pairs) whose sum is hs
template <int WT, int NCOL>
__device__ __forceinline__ float down_piece_dot_p(const DownPiece<WT, NCOL>& d, const uint32_t (&p)[8],
                                                  const uint32_t* hp, float hs) {
  float c0 = -(128.0f + (float)QOff<WT>::v) * hs, c1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    c0 = dot2_bf16(p[i], hp[i], c0);
    c1 = dot2_bf16(p[i + 1], hp[i + 1], c1);
  }
  return d.s * (c0 + c1);
}

template <int WT, int NCOL>
__device__ __forceinline__ float down_piece_dot(const DownPiece<WT, NCOL>& d, int half, const uint32_t* hp, float hs) {
  if constexpr (is_q<WT>()) {
    uint32_t p[8];
    if constexpr (WT == MOE_W_Q4) {
#pragma unroll
      for (int w = 0; w < 2; w++)
#pragma unroll
        for (int s = 0; s < 4; s++) p[4 * w + s] = ((d.w[w] >> (4 * s)) & 0x000F000Fu) | BF16_MAGIC2;
    } else {
      // pairs 8*half + i: low bits from L(half) bits 2i, high bits from HB bits 8*half + i (+16)
      const uint32_t hsh = d.w[1] >> (8 * half);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t v = ((d.w[0] >> (2 * i)) & 0x00030003u) | BF16_MAGIC2;
        const uint32_t h = (i >= 2) ? (hsh >> (i - 2)) : (hsh << (2 - i));
        p[i] = v | (h & 0x00040004u);
      }
    }
    float c0 = -(128.0f + (float)QOff<WT>::v) * hs, c1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      c0 = dot2_bf16(p[i], hp[i], c0);
      c1 = dot2_bf16(p[i + 1], hp[i + 1], c1);
    }
    return d.s * (c0 + c1);
  } else if constexpr (WT == MOE_W_BF16) {
    float c0 = 0.0f, c1 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCOL / 2; i += 2) {
      c0 = dot2_bf16(d.w[i], hp[i], c0);
      c1 = dot2_bf16(d.w[i + 1], hp[i + 1], c1);
    }
    return c0 + c1;
  } else {
    float c0 = 0.0f, c1 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCOL / 2; i++) {
      c0 = __builtin_fmaf(__uint_as_float(d.w[2 * i]), bf16_lo(hp[i]), c0);
      c1 = __builtin_fmaf(__uint_as_float(d.w[2 * i + 1]), bf16_hi(hp[i]), c1);
    }
    return c0 + c1;
  }
}

// ---------------------------------------------------------------------------
// Kernel A: router rows (blocks < nRB) and shared-expert column groups
// ---------------------------------------------------------------------------
constexpr int A_CPR = 8;  // router float4 chunks per lane and batch
constexpr int A_RPT = 4;  // shared down rows per thread and batch

template <int SWT, int MAXB>
__global__ __launch_bounds__(DA_THREADS) void k_dec_a(LayerDev L, const uint16_t* __restrict__ x, int B, DecodeWs ws,
                                                      int nRB, int rg) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = L.H, E = L.E, I = L.I;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  if ((int)blockIdx.x < nRB) {
    const int e = blockIdx.x * 8 + wave;
    const bool valid = e < E;
    const int n4 = H >> 2;
    const float4* wr = reinterpret_cast<const float4*>(L.router_w + (size_t)(valid ? e : 0) * H);
    const double bias = (valid && L.router_b) ? (double)L.router_b[e] : 0.0;
    double acc[MAXB];
#pragma unroll
    for (int t = 0; t < MAXB; t++) acc[t] = 0.0;
    for (int c0 = 0; c0 < n4; c0 += 64 * A_CPR) {
      float4 w[A_CPR];
      // loads with clamped indices and no branch (a load inside a branch makes
      // the compiler wait for every load in flight where the branch joins);
      // elements past the row are masked after
#pragma unroll
      for (int i = 0; i < A_CPR; i++) w[i] = wr[min(c0 + lane + 64 * i, n4 - 1)];
#pragma unroll
      for (int i = 0; i < A_CPR; i++)
        if (!(valid && c0 + lane + 64 * i < n4)) w[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 == 0) {
        stage_tokens<DA_THREADS>(x, B, H, xs, nullptr);
        __syncthreads();
      }
#pragma unroll
      for (int t = 0; t < MAXB; t++) {
        if (t < B) {
#pragma unroll
          for (int i = 0; i < A_CPR; i++) {
            const int c = c0 + lane + 64 * i;
            if (c < n4) {
              const uint2 xv = *reinterpret_cast<const uint2*>(xs + (size_t)t * H + 4 * c);
              acc[t] = __builtin_fma((double)w[i].x, (double)bf16_lo(xv.x), acc[t]);
              acc[t] = __builtin_fma((double)w[i].y, (double)bf16_hi(xv.x), acc[t]);
              acc[t] = __builtin_fma((double)w[i].z, (double)bf16_lo(xv.y), acc[t]);
              acc[t] = __builtin_fma((double)w[i].w, (double)bf16_hi(xv.y), acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < B) {
        const double tot = wave_total_f64(acc[t]);
        if (valid && lane == 0) ws.logits[(size_t)t * E + e] = tot + bias;
      }
    }
    return;
  }
  // ---- shared expert: intermediate columns 8p .. 8p+7 (p = workgroup index)
  constexpr int KC = kchunk<SWT>();
  constexpr int SCPT = 8;  // gate/up chunks per lane and batch (32 K parts x 8 = 256 chunks)
  const int R = 2 * I;
  const int p = blockIdx.x - nRB;
  const int q = p >> 1, j0 = (p & 1) * 8;
  // lane -> (row r = lane / 4: 0..7 gate rows j0.., 8..15 up rows; kpart = lane % 4 + 4 wave):
  // the eight gate (up) rows are consecutive, so a load reads 8 x 16 B in a row
  const int r = lane >> 2;
  const int row = 32 * q + (r < 8 ? j0 + r : 16 + j0 + (r - 8));
  const int kp = (lane & 3) + 4 * wave;
  const int nc = H / KC;
  float* s_gu = reinterpret_cast<float*>(smem + (size_t)B * H * 2);  // [8 waves][MAXB][16 rows]
  uint32_t* s_hp = reinterpret_cast<uint32_t*>(s_gu + 8 * MAXB * 16);  // [MAXB][4] bf16 pairs
  float* s_hs = reinterpret_cast<float*>(s_hp + MAXB * 4);             // [MAXB]
  const int col0 = 8 * p;
  // first batch of down pieces is issued together with the gate/up loads
  DownPiece<SWT, 8> dp[A_RPT];
#pragma unroll
  for (int i = 0; i < A_RPT; i++)  // clamped, unconditional (rows past H are not used)
    load_down_piece<SWT, 8>(L.sdn, nullptr, H, min((int)threadIdx.x + DA_THREADS * i, H - 1), col0, dp[i]);
  float acc[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += 32 * SCPT) {
    Raw raw[SCPT];
#pragma unroll
    for (int i = 0; i < SCPT; i++)  // clamped, unconditional (chunks past the row are not used)
      raw[i] = load_chunk<SWT>(L.sgu, (size_t)min(c0 + kp + 32 * i, nc - 1) * R + row);
    if (c0 == 0) {
      stage_tokens<DA_THREADS>(x, B, H, xs, nullptr);
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < B) {
#pragma unroll
        for (int i = 0; i < SCPT; i++) {
          const int c = c0 + kp + 32 * i;
          if (c < nc) acc[t] = ddot<SWT>(raw[i], xs + (size_t)t * H + (size_t)c * KC, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    if (t < B) {
      float v = acc[t];
      v += dpp_f32<DPP_XOR1>(v);  // the row's four K-part lanes, fixed order
      v += dpp_f32<DPP_XOR2>(v);
      if ((lane & 3) == 0) s_gu[(wave * MAXB + t) * 16 + r] = v;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < B * 8) {
    const int t = threadIdx.x >> 3, j = threadIdx.x & 7;
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int wv = 0; wv < 8; wv++) {
      g += s_gu[(wv * MAXB + t) * 16 + j];
      u += s_gu[(wv * MAXB + t) * 16 + 8 + j];
    }
    reinterpret_cast<uint16_t*>(s_hp)[t * 8 + j] = f32_to_bf16(silu_f32(g) * u);
  }
  __syncthreads();
  if ((int)threadIdx.x < B) {
    const uint16_t* hh = reinterpret_cast<const uint16_t*>(s_hp) + threadIdx.x * 8;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) sum += bf16_to_f32(hh[j]);
    s_hs[threadIdx.x] = sum;
  }
  __syncthreads();
  const size_t pbase = (size_t)B * L.k * rg;  // shared partials follow the routed ones (rg groups per slot)
  for (int r0 = 0; r0 < H; r0 += DA_THREADS * A_RPT) {
    if (r0 > 0) {
#pragma unroll
      for (int i = 0; i < A_RPT; i++)
        load_down_piece<SWT, 8>(L.sdn, nullptr, H, min(r0 + (int)threadIdx.x + DA_THREADS * i, H - 1), col0, dp[i]);
    }
#pragma unroll
    for (int i = 0; i < A_RPT; i++) {
      const int rw = r0 + threadIdx.x + DA_THREADS * i;
      if (rw < H) {
#pragma unroll
        for (int t = 0; t < MAXB; t++) {
          if (t < B) {
            const float v = down_piece_dot<SWT, 8>(dp[i], 0, s_hp + 4 * t, s_hs[t]);
            ws.part[(pbase + (size_t)t * (I >> 3) + p) * H + rw] = v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Routing of the batch (one workgroup): top-k of each token (one wave per
// token) and the unique experts of the batch in first-occurrence (slot)
// order with the tokens using each, written to the workspace for kernel B.
// Route record: [0] unique count, then idx[MAXB*16], gate bits[MAXB*16],
// unique experts[MAXB*16], token masks[MAXB*16].
// ---------------------------------------------------------------------------
constexpr int ROUTE_MAXS = 8 * 16;  // slots of the largest batch
__device__ __forceinline__ int32_t* route_idx(int32_t* r) { return r + 4; }
__device__ __forceinline__ int32_t* route_gate(int32_t* r) { return r + 4 + ROUTE_MAXS; }
__device__ __forceinline__ int32_t* route_uniq(int32_t* r) { return r + 4 + 2 * ROUTE_MAXS; }
__device__ __forceinline__ int32_t* route_mask(int32_t* r) { return r + 4 + 3 * ROUTE_MAXS; }

template <int MAXB>
__global__ __launch_bounds__(DB_THREADS) void k_dec_route(int E, int k, int B, DecodeWs ws, int32_t* idx_out,
                                                          float* gate_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int s_idx[MAXB * 16];
  __shared__ float s_gate[MAXB * 16];
  __shared__ int s_uid[MAXB * 16];
  __shared__ uint32_t s_msk[MAXB * 16];
  __shared__ int s_wcnt[DB_THREADS / 64];
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tks = smem;                        // [B] top-k scratch
  int* mark = reinterpret_cast<int*>(smem);   // reuses it after the top-k
  int32_t* rt = ws.route;
  double lv[16];
  const int tw = wave;  // B <= 8 = waves: one token per wave
#pragma unroll
  for (int i = 0; i < 16; i++)  // clamped, unconditional; masked after
    lv[i] = ws.logits[(size_t)min(tw, B - 1) * E + min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < 16; i++)
    if (!(tw < B && lane + 64 * i < E)) lv[i] = -__builtin_inf();
  if (tw < B) {
    int mi;
    float mg;
    wave_topk(lv, E, k, lane, tks + (size_t)tw * TOPK_SCRATCH, mi, mg);
    if (lane < k) {
      s_idx[tw * k + lane] = mi;
      s_gate[tw * k + lane] = mg;
    }
  }
  __syncthreads();
  const int nslot = B * k;
  for (int i = threadIdx.x; i < nslot; i += DB_THREADS) {
    route_idx(rt)[i] = s_idx[i];
    route_gate(rt)[i] = __float_as_int(s_gate[i]);
    if (idx_out) idx_out[i] = s_idx[i];
    if (gate_out) gate_out[i] = s_gate[i];
  }
  if constexpr (MAXB == 1) {
    if ((int)threadIdx.x < k) {
      route_uniq(rt)[threadIdx.x] = s_idx[threadIdx.x];
      route_mask(rt)[threadIdx.x] = 1;
    }
    if (threadIdx.x == 0) rt[0] = k;
  } else {
    for (int e = threadIdx.x; e < E; e += DB_THREADS) mark[e] = 0x7FFFFFFF;
    __syncthreads();
    if ((int)threadIdx.x < nslot) atomicMin(&mark[s_idx[threadIdx.x]], (int)threadIdx.x);
    __syncthreads();
    const bool first = (int)threadIdx.x < nslot && mark[s_idx[threadIdx.x]] == (int)threadIdx.x;
    const uint64_t bal = __ballot(first);
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int wv = 0; wv < wave; wv++) base += s_wcnt[wv];
    const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
    if (first) s_uid[threadIdx.x] = rank;
    if ((int)threadIdx.x < nslot) s_msk[threadIdx.x] = 0u;
    __syncthreads();
    // each unique expert's token mask: the bits of the tokens that chose it
    if ((int)threadIdx.x < nslot) {
      const int u = s_uid[mark[s_idx[threadIdx.x]]];
      if (first) route_uniq(rt)[u] = s_idx[threadIdx.x];
      atomicOr(&s_msk[u], 1u << (threadIdx.x / k));
    }
    __syncthreads();
    if ((int)threadIdx.x < nslot) route_mask(rt)[threadIdx.x] = (int32_t)s_msk[threadIdx.x];
    if (threadIdx.x == 0) {
      int n = 0;
      for (int wv = 0; wv < DB_THREADS / 64; wv++) n += s_wcnt[wv];
      rt[0] = n;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel B: routed experts, one (unique expert, column group) each
// ---------------------------------------------------------------------------
constexpr int B_CPT = 4;  // gate/up chunks per lane and batch
constexpr int B_RPT = 4;  // down rows per thread and batch

// Kernel B: one workgroup per (unique expert u, group q of GCOL intermediate
// columns). Quantised weights take GCOL = 32 (or 64): the workgroup streams
// the 2 GCOL gate/up rows and whole chunks of each down row, so a call has
// half (a quarter) of the workgroups and of the partial products that
// 16-column groups give; dense weights take GCOL = 16 (a wider dense down row
// would not fit the registers).
//   gate/up: wave w owns rows GCOL/4 w .. (+GCOL/4) of the group, 64/(GCOL/4)
//   lanes per row split the K chunks; two batches of chunk loads in flight.
//   down: rows tid + 512 i, i < B_RPT, per pass over H.
template <int WT, int MAXB, int GCOL>
__global__ __launch_bounds__(DB_THREADS) void k_dec_b(LayerDev L, const uint16_t* __restrict__ x, int B, DecodeWs ws) {
  static_assert(GCOL == 16 || ((GCOL == 32 || GCOL == 64) && is_q<WT>()), "whole-chunk groups for quantised weights only");
  constexpr bool WHOLE = GCOL >= 32;  // down rows as whole chunks (GCOL / 32 per row)
  constexpr int DCH = WHOLE ? GCOL / 32 : 1;
  const int H = L.H, I = L.I, k = L.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RPW = GCOL / 4;  // gate/up rows per wave
  constexpr int LPR = 64 / RPW;  // lanes (K parts) per row
  constexpr int NHS = GCOL >= 32 ? GCOL / 32 : 1;  // h block sums per token
  __shared__ int s_idx[MAXB * 16];
  __shared__ float s_gate[MAXB * 16];
  __shared__ int s_uniq[MAXB * 16];
  __shared__ uint32_t s_mask[MAXB * 16];
  __shared__ int s_nu;
  __shared__ float s_gu[MAXB * 2 * GCOL];
  __shared__ __align__(16) uint32_t s_hp[MAXB * GCOL / 2];  // h of token t: bf16 pairs at s_hp + GCOL/2 t
  __shared__ float s_hs[MAXB * NHS];
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool QT = is_q<WT>();
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)B * H * 2);

  // 1. the batch's routing (from the routing kernel)
  const int32_t* rt = ws.route;
  const int nslot = B * k;
  if ((int)threadIdx.x < nslot) {
    s_idx[threadIdx.x] = route_idx(ws.route)[threadIdx.x];
    s_gate[threadIdx.x] = __int_as_float(route_gate(ws.route)[threadIdx.x]);
    s_uniq[threadIdx.x] = route_uniq(ws.route)[threadIdx.x];
    s_mask[threadIdx.x] = (uint32_t)route_mask(ws.route)[threadIdx.x];
  }
  if (threadIdx.x == 0) s_nu = rt[0];
  __syncthreads();
  const int nu = s_nu;
  const int gpe = I / GCOL;  // column groups per expert
  const int u = blockIdx.x / gpe;
  if (u >= nu) return;  // uniform
  const int q = blockIdx.x - u * gpe;
  const int e = s_uniq[u];
  const uint32_t mask = s_mask[u];

  // 2. loads: the group's gate/up rows and its down pieces; every load of the
  //    first batches is issued before any wait (unconditional, clamped indices)
  constexpr int KC = kchunk<WT>();
  const int R = 2 * I;
  const int rr = RPW * wave + lane / LPR;
  const int row = 2 * GCOL * q + rr;
  const int kp = lane % LPR;
  const int nc = H / KC;
  const uint8_t* wgu = L.gu + (size_t)e * L.gu_stride;
  const uint16_t* wgs = QT ? L.gu_s + (size_t)e * L.gu_s_stride : nullptr;
  const uint8_t* wdn = L.dn + (size_t)e * L.dn_stride;
  const uint16_t* wds = QT ? L.dn_s + (size_t)e * L.dn_s_stride : nullptr;
  const int col0 = GCOL * q;
  // down pieces of the first pass: GCOL = 16 a half chunk per row (DownPiece),
  // GCOL = 64 two chunks per row with their scales (raw fp16 bits)
  constexpr int RPT = DCH == 2 ? 2 : B_RPT;   // down rows per thread and pass
  constexpr int CPT = WHOLE ? 2 : B_CPT;      // gate/up chunks per lane and batch (two batches in flight)
  DownPiece<WT, 16> dp[WHOLE ? 1 : B_RPT];
  Raw dr[WHOLE ? RPT : 1][DCH];
  uint16_t dsb[WHOLE ? RPT : 1][DCH];
  auto load_down = [&](int r0) {  // rows past H are not used
    if constexpr (!WHOLE) {
#pragma unroll
      for (int i = 0; i < B_RPT; i++)
        load_down_piece<WT, 16>(wdn, wds, H, min(r0 + (int)threadIdx.x + DB_THREADS * i, H - 1), col0, dp[i]);
    } else {
#pragma unroll
      for (int i = 0; i < RPT; i++) {
        const int rw = min(r0 + (int)threadIdx.x + DB_THREADS * i, H - 1);
#pragma unroll
        for (int h = 0; h < DCH; h++) {
          dr[i][h] = load_chunk<WT>(wdn, (size_t)(col0 / 32 + h) * H + rw);
          dsb[i][h] = wds[(size_t)(col0 / 32 + h) * H + rw];
        }
      }
    }
  };
  const int nb = H >> 5;
  float acc[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
  Raw raw[2][CPT];
  uint16_t sc[2][CPT];
  auto load_batch = [&](int c0, Raw (&rw)[CPT], uint16_t (&sw)[CPT]) {  // chunks past the row are not used
#pragma unroll
    for (int i = 0; i < CPT; i++) rw[i] = load_chunk<WT>(wgu, (size_t)min(c0 + kp + LPR * i, nc - 1) * R + row);
    if constexpr (QT) {
#pragma unroll
      for (int i = 0; i < CPT; i++) sw[i] = wgs[(size_t)min(c0 + kp + LPR * i, nc - 1) * R + row];
    }
  };
  auto compute_batch = [&](int c0, const Raw (&rw)[CPT], const uint16_t (&sw)[CPT]) {
    if constexpr (QT) {
      // each chunk unpacked once, then dotted with every token of the expert
#pragma unroll
      for (int i = 0; i < CPT; i++) {
        const int c = c0 + kp + LPR * i;
        if (c < nc) {
          uint32_t p[16];
          qunpack32<WT>(rw[i], p);
          const float scl = f16_to_f32(sw[i]);
#pragma unroll
          for (int t = 0; t < MAXB; t++)
            if (t < B && (mask >> t & 1u))
              acc[t] = __builtin_fmaf(scl, qdot32_p<WT>(p, xs + (size_t)t * H + 32 * c, xsum[t * nb + c]), acc[t]);
        }
      }
    } else {
      (void)sw;
#pragma unroll
      for (int t = 0; t < MAXB; t++) {
        if (t < B && (mask >> t & 1u)) {
#pragma unroll
          for (int i = 0; i < CPT; i++) {
            const int c = c0 + kp + LPR * i;
            if (c < nc) acc[t] = ddot<WT>(rw[i], xs + (size_t)t * H + (size_t)c * KC, acc[t]);
          }
        }
      }
    }
  };
  constexpr int CPB = LPR * CPT;  // chunks per batch of the workgroup's rows
  load_batch(0, raw[0], sc[0]);
  if constexpr (!WHOLE) load_down(0);  // whole chunks: after the gate/up rows (registers)
  if (CPB < nc) load_batch(CPB, raw[1], sc[1]);
  // the activations of this expert's tokens only (a token's row at xs + t H),
  // with their 32-element block sums, while the weights are in flight
  {
    const int na = __popc(mask & ((1u << B) - 1u));
    const int n16 = H / 8;
    for (int i = threadIdx.x; i < na * n16; i += DB_THREADS) {
      const int a = i / n16;
      uint32_t m = mask;
      for (int j = 0; j < a; j++) m &= m - 1u;  // drop the a lowest tokens
      const int t = __ffs(m) - 1;
      const int c = i - a * n16;
      reinterpret_cast<uint4*>(xs + (size_t)t * H)[c] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[c];
    }
    if (QT) {
      __syncthreads();
      for (int i = threadIdx.x; i < B * nb; i += DB_THREADS) {
        const int t = i / nb;
        if (mask >> t & 1u) {
          const uint32_t* v = reinterpret_cast<const uint32_t*>(xs + (size_t)i * 32);
          float sum = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; j++) sum += bf16_lo(v[j]) + bf16_hi(v[j]);
          xsum[i] = sum;
        }
      }
    }
    __syncthreads();
  }
  // batches two at a time: batch n + 2 is issued before batch n + 1 is computed
  for (int c0 = 0; c0 < nc; c0 += 2 * CPB) {
    compute_batch(c0, raw[0], sc[0]);
    if (c0 + 2 * CPB < nc) load_batch(c0 + 2 * CPB, raw[0], sc[0]);
    if (c0 + CPB < nc) {
      compute_batch(c0 + CPB, raw[1], sc[1]);
      if (c0 + 3 * CPB < nc) load_batch(c0 + 3 * CPB, raw[1], sc[1]);
    }
  }
  if constexpr (WHOLE) load_down(0);  // in flight through the SwiGLU below
  // fold the LPR lanes of each row (fixed order)
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    if (t < B && (mask >> t & 1u)) {
      float v = acc[t];
      static_assert(LPR == 16 || LPR == 8 || LPR == 4, "lanes per row");
      if constexpr (LPR == 16) {
        v = sum16_f32(v);
      } else if constexpr (LPR == 8) {
        v = sum8_f32(v);
      } else {
        v += dpp_f32<DPP_XOR1>(v);
        v += dpp_f32<DPP_XOR2>(v);
      }
      if (kp == 0) s_gu[t * 2 * GCOL + rr] = v;
    }
  }
  __syncthreads();
  // 3. SwiGLU (bf16 h) and the block sums of h; intermediate j of the group:
  //    gate row 32 (j / 16) + j % 16, up row + 16
  for (int i = threadIdx.x; i < MAXB * GCOL; i += DB_THREADS) {
    const int t = i / GCOL, j = i % GCOL;
    if (t < B && (mask >> t & 1u)) {
      const int gr = 32 * (j >> 4) + (j & 15);
      reinterpret_cast<uint16_t*>(s_hp)[t * GCOL + j] =
          f32_to_bf16(silu_f32(s_gu[t * 2 * GCOL + gr]) * s_gu[t * 2 * GCOL + gr + 16]);
    }
  }
  __syncthreads();
  {
    // sums of 16 (GCOL = 16) or 32 (GCOL = 64) consecutive bf16 h values: one
    // group of 16 lanes per sum, fixed order
    constexpr int HG = GCOL >= 32 ? 32 : 16;
    const int g = threadIdx.x >> 4, j = threadIdx.x & 15;
    const int t = g / NHS, hb = g % NHS;
    float hv = 0.0f;
    const bool act = g < MAXB * NHS && t < B && (mask >> t & 1u);
    if (act) {
      const uint16_t* hh = reinterpret_cast<const uint16_t*>(s_hp) + t * GCOL + HG * hb;
      hv = bf16_to_f32(hh[j]);
      if constexpr (HG == 32) hv += bf16_to_f32(hh[j + 16]);
    }
    hv = sum16_f32(hv);
    if (act && j == 0) s_hs[t * NHS + hb] = hv;
  }
  __syncthreads();
  // 4. gated partial down products of this expert's tokens
  int slot[MAXB];
  float gt[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    slot[t] = -1;
    gt[t] = 0.0f;
    if (t < B && (mask >> t & 1u)) {
      for (int j = 0; j < k; j++)
        if (s_idx[t * k + j] == e) {
          slot[t] = t * k + j;
          gt[t] = s_gate[t * k + j];
        }
    }
  }
  for (int r0 = 0; r0 < H; r0 += DB_THREADS * RPT) {
    if (r0 > 0) load_down(r0);
#pragma unroll
    for (int i = 0; i < RPT; i++) {
      const int rw = r0 + threadIdx.x + DB_THREADS * i;
      if (rw < H) {
        if constexpr (WHOLE) {
          uint32_t pc[DCH][16];  // the row's chunks unpacked once for all tokens
          float sd[DCH];
#pragma unroll
          for (int h = 0; h < DCH; h++) {
            qunpack32<WT>(dr[i][h], pc[h]);
            sd[h] = f16_to_f32(dsb[i][h]);
          }
#pragma unroll
          for (int t = 0; t < MAXB; t++) {
            if (slot[t] >= 0) {
              const uint16_t* ht = reinterpret_cast<const uint16_t*>(s_hp) + t * GCOL;
              float v = sd[0] * qdot32_p<WT>(pc[0], ht, s_hs[t * NHS]);
              if constexpr (DCH == 2) v += sd[1] * qdot32_p<WT>(pc[1], ht + 32, s_hs[t * NHS + 1]);
              ws.part[((size_t)slot[t] * gpe + q) * H + rw] = gt[t] * v;
            }
            // one token's h (32 registers) at a time: hoisting the reads of
            // every token would not fit the registers
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          uint32_t p[8];
          if constexpr (QT) down_piece_unpack<WT, 16>(dp[i], q & 1, p);  // once for all tokens
#pragma unroll
          for (int t = 0; t < MAXB; t++) {
            if (slot[t] >= 0) {
              float v;
              if constexpr (QT) v = down_piece_dot_p<WT, 16>(dp[i], p, s_hp + 8 * t, s_hs[t]);
              else v = down_piece_dot<WT, 16>(dp[i], q & 1, s_hp + 8 * t, s_hs[t]);
              ws.part[((size_t)slot[t] * gpe + q) * H + rw] = gt[t] * v;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel C: y[t][r] = sum over token t's partials (routed slots in order,
// their column groups in order, then the shared expert's 8-column groups)
// ---------------------------------------------------------------------------
constexpr int DC_BATCH = 24;  // partial loads in flight per thread

__global__ __launch_bounds__(DC_THREADS) void k_dec_c(const float* __restrict__ part, int H, int k, int I, int B,
                                                      uint16_t* __restrict__ y, int has_shared, int rg) {
  __shared__ float red[DC_SPLIT][DC_ROWS];
  const int t = blockIdx.y;
  const int rr = threadIdx.x % DC_ROWS, sp = threadIdx.x / DC_ROWS;
  const int r = blockIdx.x * DC_ROWS + rr;
  const int nr = k * rg;  // routed partials of this token (rg column groups per slot), then its shared-expert partials
  const int ns = has_shared ? (I >> 3) : 0;
  const size_t rbase = (size_t)t * nr;
  const size_t sbase = (size_t)B * nr + (size_t)t * ns;
  const int n = nr + ns;
  float acc = 0.0f;
  if (r < H) {
    // this thread's partials: i = sp, sp + SPLIT, ... (all loads of a batch issued together)
    for (int i0 = sp; i0 < n; i0 += DC_SPLIT * DC_BATCH) {
      float v[DC_BATCH];
#pragma unroll
      for (int j = 0; j < DC_BATCH; j++) {
        const int i = i0 + DC_SPLIT * j;
        const size_t pi = (i < nr) ? rbase + i : sbase + (i - nr);
        v[j] = (i < n) ? part[pi * H + r] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < DC_BATCH; j++) acc += v[j];
    }
  }
  red[sp][rr] = acc;
  __syncthreads();
  if (sp == 0 && r < H) {
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < DC_SPLIT; j++) sum += red[j][rr];
    y[(size_t)t * H + r] = f32_to_bf16(sum);
  }
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
size_t decode_lds_b(int wt, int B, int H, int E, int k) {
  (void)E; (void)k;
  const bool q = (wt == MOE_W_Q4 || wt == MOE_W_Q3);
  const size_t xsb = q ? (size_t)((B * (H / 32) + 1) & ~1) * 4 : 0;
  return (size_t)B * H * 2 + xsb;
}

template <int WT, int SWT, int MAXB>
static hipError_t launch_t(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out, float* gate_out,
                           const DecodeWs& ws, hipStream_t st) {
  const int H = L.H, I = L.I, E = L.E, k = L.k;
  constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
  // kernel B's intermediate columns per workgroup (and per routed partial):
  // one whole chunk per down row for quantised weights (measured at B = 4 and
  // 8 on the Zipf-routed Q3 layer: 32 columns beat 16 and 64; 64 makes the
  // workgroups of an expert chosen by every token of the batch the long pole)
  constexpr int gcol = is_q<WT>() ? 32 : 16;
  const int rg = I / gcol;
  {
    const int nRB = (E + 7) / 8;
    const int nSB = (SWT == MOE_W_NONE) ? 0 : I / 8;
    const size_t lds = (size_t)B * H * 2 + (size_t)(8 * MAXB * 16 + MAXB * 4 + MAXB) * 4;
    (void)launch_k(KC_DEC_ROUTER_SHARED, (k_dec_a<SW, MAXB>), dim3(nRB + nSB), dim3(DA_THREADS), lds, st, L, x, B, ws, nRB,
                   rg);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const size_t tk = (size_t)B * TOPK_SCRATCH, mk = (size_t)E * 4;
    (void)launch_k(KC_DEC_ROUTE, (k_dec_route<MAXB>), dim3(1), dim3(DB_THREADS), tk > mk ? tk : mk, st, E, k, B, ws,
                   idx_out, gate_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int maxU = (B * k < E) ? B * k : E;
    const size_t lds = decode_lds_b(WT, B, H, E, k);
    (void)launch_k(KC_DEC_GATE_UP, (k_dec_b<WT, MAXB, gcol>), dim3(maxU * rg), dim3(DB_THREADS), lds, st, L, x, B, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  (void)launch_k(KC_DEC_DOWN, k_dec_c, dim3((H + DC_ROWS - 1) / DC_ROWS, B), dim3(DC_THREADS), 0, st, ws.part, H, k, I, B, y,
                 SWT == MOE_W_NONE ? 0 : 1, rg);
  return hipGetLastError();
}

template <int WT, int SWT>
static hipError_t launch_b(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                           const DecodeWs& ws, hipStream_t st) {
  if (B == 1) return launch_t<WT, SWT, 1>(L, x, B, y, io, go, ws, st);
  return launch_t<WT, SWT, 8>(L, x, B, y, io, go, ws, st);
}

template <int WT>
static hipError_t launch_s(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                           const DecodeWs& ws, hipStream_t st) {
  switch (L.swt) {
    case MOE_W_BF16: return launch_b<WT, MOE_W_BF16>(L, x, B, y, io, go, ws, st);
    case MOE_W_F32: return launch_b<WT, MOE_W_F32>(L, x, B, y, io, go, ws, st);
    default: return launch_b<WT, MOE_W_NONE>(L, x, B, y, io, go, ws, st);
  }
}

// One stack layer at decode: the one-kernel path with the norm and the
// residual inside when batch 1 fits there, else RMSNorm, the decode kernels
// and the residual add in turn (z and y in the caller's buffers or the
// workspace's).
hipError_t launch_stack_decode(const LayerDev& L, uint16_t* h, int B, float eps, uint16_t* z_out, uint16_t* y_out,
                               int32_t* idx_out, float* gate_out, const DecodeWs& ws, hipStream_t st) {
  if (B == 1 && decode1_fits(L.E, L.H, L.I, L.k, L.swt != MOE_W_NONE)) {
    const StackIo S{h, z_out, y_out, eps};
    return launch_decode_fused(L, nullptr, nullptr, idx_out, gate_out, ws, st, &S);
  }
  uint16_t* z = z_out ? z_out : ws.zb;
  uint16_t* y = y_out ? y_out : ws.yb;
  hipError_t e = launch_rmsnorm(h, z, B, L.H, eps, st);
  if (e != hipSuccess) return e;
  e = launch_decode(L, z, B, y, idx_out, gate_out, ws, st);
  if (e != hipSuccess) return e;
  return launch_residual(h, y, B, L.H, st);
}

hipError_t launch_decode(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out, float* gate_out,
                         const DecodeWs& ws, hipStream_t st) {
  if (B == 1 && decode1_fits(L.E, L.H, L.I, L.k, L.swt != MOE_W_NONE))
    return launch_decode_fused(L, x, y, idx_out, gate_out, ws, st);
  if (B > 1 && decode1b_fits(L.wt, L.E, L.H, L.I, L.k, L.swt != MOE_W_NONE, B))
    return launch_decode_fused_b(L, x, B, y, idx_out, gate_out, ws, st);
  switch (L.wt) {
    case MOE_W_Q4: return launch_s<MOE_W_Q4>(L, x, B, y, idx_out, gate_out, ws, st);
    case MOE_W_Q3: return launch_s<MOE_W_Q3>(L, x, B, y, idx_out, gate_out, ws, st);
    case MOE_W_BF16: return launch_s<MOE_W_BF16>(L, x, B, y, idx_out, gate_out, ws, st);
    default: return launch_s<MOE_W_F32>(L, x, B, y, idx_out, gate_out, ws, st);
  }
}

}  // namespace moe
