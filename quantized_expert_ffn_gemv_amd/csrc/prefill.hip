// Prefill path: T tokens through one MoE layer.
//
//   k_pf_router      router logits, fp64 accumulation (LDS-tiled)
//   k_pf_topk        ordered top-k and renormalised gates, one wave per token
//   k_pf_count       per-block expert histograms (LDS atomics: order-free)
//   k_pf_scan        exclusive scans: expert offsets, per-block bases, GEMM tiles
//   k_pf_scatter     stable permutation: slots sorted by expert, token order
//                    kept inside an expert (wave ballots, no float atomics)
//   k_pf_gemm<...>   MFMA grouped GEMM. Gate/up: each expert's gathered token
//                    rows x the expert's fused gate/up weights, dequantised
//                    to bf16 in LDS, SwiGLU epilogue -> h (sorted order).
//                    Down: h rows x dequantised down weights -> Y (sorted).
//                    The shared expert runs through the same kernel as one
//                    more "expert" that owns every token.
//   k_pf_combine     y[t] = sum_j gate[t][j] * Y[inv[t,j]] + Ys[t], slot order
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router: logits[t][e] = sum_h W[e][h] x[t][h] + b[e] in fp64
// ---------------------------------------------------------------------------
constexpr int RT_M = 64, RT_N = 64, RT_K = 16;

__global__ __launch_bounds__(256) void k_pf_router(const float* __restrict__ W, const float* __restrict__ bias,
                                                    const uint16_t* __restrict__ x, int T, int E, int H,
                                                    double* __restrict__ logits) {
  __shared__ double sa[RT_K][RT_M + 1];
  __shared__ double sb[RT_K][RT_N + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * RT_M, n0 = blockIdx.y * RT_N;
  const int tm = tid / 16, tn = tid % 16;  // 4x4 outputs each: rows tm + 16 i, cols tn + 16 j
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = 0.0;
  for (int k0 = 0; k0 < H; k0 += RT_K) {
    // 64 x 16 of each operand: 1024 values, 4 per thread
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = tid + 256 * r;
      const int row = i / RT_K, kk = i % RT_K;
      const int t = m0 + row, e = n0 + row;
      sa[kk][row] = (t < T) ? (double)bf16_to_f32(x[(size_t)t * H + k0 + kk]) : 0.0;
      sb[kk][row] = (e < E) ? (double)W[(size_t)e * H + k0 + kk] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < RT_K; kk++) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; i++) a[i] = sa[kk][tm + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; j++) b[j] = sb[kk][tn + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = m0 + tm + 16 * i;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = n0 + tn + 16 * j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? (double)bias[e] : 0.0);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_topk(const double* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ idx, float* __restrict__ gates,
                                                  int32_t* idx_out, float* gate_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double* l = logits + (size_t)t * E;
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? l[e] : -__builtin_inf();
  }
  double m = 0.0, myv = -__builtin_inf();
  int myi = 0;
  for (int r = 0; r < k; r++) {
    double best = -__builtin_inf();
    int bi = 0x7FFFFFFF;
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
  const double ev = (lane < k) ? exp(myv - m) : 0.0;
  const double z = wave_sum_f64(ev);
  if (lane < k) {
    const float g = (float)(ev / z);
    idx[(size_t)t * k + lane] = myi;
    gates[(size_t)t * k + lane] = g;
    if (idx_out) idx_out[(size_t)t * k + lane] = myi;
    if (gate_out) gate_out[(size_t)t * k + lane] = g;
  }
}

// ---------------------------------------------------------------------------
// Histogram / scan / stable permutation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_count(const int32_t* __restrict__ idx, int T, int E, int k,
                                                   int32_t* __restrict__ blk_counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * PF_TOK_PER_BLK;
  const int t1 = min(T, t0 + PF_TOK_PER_BLK);
  for (int s = t0 * k + threadIdx.x; s < t1 * k; s += 256) atomicAdd(&hist[idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_pf_scan(const int32_t* __restrict__ blk_counts, int nblk, int E,
                                                   int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ tile_start,
                                                   int32_t* counts_out) {
  __shared__ int s_tot[1024];
  __shared__ int s_til[1024];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E)
    for (int b = 0; b < nblk; b++) tot += blk_counts[(size_t)b * E + e];
  s_tot[e] = (e < E) ? tot : 0;
  s_til[e] = (e < E) ? (tot + PF_BM - 1) / PF_BM : 0;
  __syncthreads();
  // inclusive Hillis-Steele scans over 1024 entries
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = (e >= o) ? s_tot[e - o] : 0;
    const int c = (e >= o) ? s_til[e - o] : 0;
    __syncthreads();
    s_tot[e] += a;
    s_til[e] += c;
    __syncthreads();
  }
  if (e < E) {
    const int off = s_tot[e] - tot;
    counts[e] = tot;
    offsets[e] = off;
    tile_start[e] = s_til[e] - (tot + PF_BM - 1) / PF_BM;
    if (counts_out) counts_out[e] = tot;
    int run = off;
    for (int b = 0; b < nblk; b++) {
      blk_base[(size_t)b * E + e] = run;
      run += blk_counts[(size_t)b * E + e];
    }
    if (e == E - 1) {
      offsets[E] = s_tot[e];
      tile_start[E] = s_til[e];
    }
  }
}

// Positions of the slots of one token block, in slot order within each expert.
__global__ __launch_bounds__(256) void k_pf_scatter(const int32_t* __restrict__ idx, int T, int E, int k,
                                                     const int32_t* __restrict__ blk_base, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
  extern __shared__ int cnt[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = blk_base[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const int t0 = blockIdx.x * PF_TOK_PER_BLK;
  const int t1 = min(T, t0 + PF_TOK_PER_BLK);
  const int s0 = t0 * k, s1 = t1 * k;
  int ebits = 0;
  while ((1 << ebits) < E) ebits++;
  for (int base = s0; base < s1; base += 256) {
    const int s = base + threadIdx.x;
    const bool act = s < s1;
    const int e = act ? idx[s] : 0;
    // lanes of this wave with the same expert
    uint64_t peers = __ballot(act);
    for (int b = 0; b < ebits; b++) {
      const uint64_t m = __ballot(act && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    if (!act) peers = 0;
    const int before = __popcll(peers & ((1ull << lane) - 1ull));
    const bool leader = act && before == 0;
    // waves in order, so earlier slots get earlier positions
    for (int w = 0; w < 4; w++) {
      if (wave == w && act) {
        const int pos = cnt[e] + before;
        perm[pos] = s;
        inv[s] = pos;
      }
      __syncthreads();
      if (wave == w && leader) cnt[e] += __popcll(peers);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM (MFMA 16x16x32 bf16, fp32 accumulate)
// ---------------------------------------------------------------------------
constexpr int G_THREADS = 256;
constexpr int G_BN = 256;       // weight rows (output columns) per tile
constexpr int G_BK = 32;        // one quantisation block per K-step
constexpr int G_LDA = 40;       // LDS row stride in bf16 (80 B: 16-byte aligned, bank-spread)
constexpr int G_MSUB = PF_BM / 16;

enum GemmKind { GK_GATE_UP = 0, GK_DOWN = 1 };

struct GemmArgs {
  // weights of expert 0 (routed) or the shared expert; chunk-major [K/kc][N][cb]
  const uint8_t* w;
  const uint16_t* ws;     // scales [K/32][N]
  size_t w_stride, ws_stride;  // per expert
  int N, K;               // weight rows, reduction length
  // A rows
  const uint16_t* a;      // gate/up: x [T][H]; down: h [rows][I]
  const int32_t* perm;    // gate/up routed: sorted position -> slot (token = slot / k); NULL = identity
  int k;
  // routed tiling (NULL offsets => single "expert" owning rows 0..M_total)
  const int32_t* offsets;     // [E+1]
  const int32_t* tile_start;  // [E+1]
  int E;
  int M_total;            // rows when offsets == NULL
  uint16_t* out;          // gate/up: h [rows][N/2]; down: Y [rows][N]
};

// Raw bytes of one 32-element K-step of weight row n (and its scale).
template <int WT>
__device__ __forceinline__ void load_b_chunk(const GemmArgs& g, const uint8_t* w, const uint16_t* ws, int n, int s,
                                             uint32_t (&raw)[32], float& scale) {
  if constexpr (WT == MOE_W_Q4) {
    const uint4 v = *reinterpret_cast<const uint4*>(w + ((size_t)s * g.N + n) * 16);
    raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
    scale = f16_to_f32(ws[(size_t)s * g.N + n]);
  } else if constexpr (WT == MOE_W_Q3) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(w + ((size_t)s * g.N + n) * 12);
    raw[0] = p[0]; raw[1] = p[1]; raw[2] = p[2];
    scale = f16_to_f32(ws[(size_t)s * g.N + n]);
  } else {
    constexpr int NCH = (WT == MOE_W_BF16) ? 4 : 8;  // 16-byte chunks per K-step
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const uint4 v = *reinterpret_cast<const uint4*>(w + ((size_t)(NCH * s + c) * g.N + n) * 16);
      raw[4 * c] = v.x; raw[4 * c + 1] = v.y; raw[4 * c + 2] = v.z; raw[4 * c + 3] = v.w;
    }
    scale = 0.0f;
  }
}

// Raw K-step -> 16 bf16 pairs (elements 2i, 2i+1 in pair i).
template <int WT>
__device__ __forceinline__ void dequant_b_chunk(const uint32_t (&raw)[32], float scale, uint32_t (&out)[16]) {
  if constexpr (WT == MOE_W_Q4 || WT == MOE_W_Q3) {
    uint32_t p[16];
    if constexpr (WT == MOE_W_Q4) {
      q4_pairs<F16_MAGIC2>(make_uint4(raw[0], raw[1], raw[2], raw[3]), p);
    } else {
      q3_pairs<F16_MAGIC2>(raw[0], raw[1], raw[2], p);
    }
    const float negbase = -(1024.0f + (float)QOff<WT>::v) * scale;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      float lo, hi;
      f16pair_dequant(p[i], scale, negbase, lo, hi);
      out[i] = pack_bf16x2(lo, hi);
    }
  } else if constexpr (WT == MOE_W_BF16) {
#pragma unroll
    for (int i = 0; i < 16; i++) out[i] = raw[i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) out[i] = pack_bf16x2(__uint_as_float(raw[2 * i]), __uint_as_float(raw[2 * i + 1]));
  }
}

template <int WT, int KIND>
__global__ __launch_bounds__(G_THREADS) void k_pf_gemm(GemmArgs g) {
  __shared__ __align__(16) uint16_t sA[PF_BM * G_LDA];
  __shared__ __align__(16) uint16_t sB[G_BN * G_LDA];
  __shared__ int s_row[PF_BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- which expert / rows
  int e = 0, m0 = 0, M = 0, pos0 = 0;
  if (g.offsets) {
    const int tile = blockIdx.x;
    if (tile >= g.tile_start[g.E]) return;
    int lo = 0, hi = g.E - 1;  // largest e with tile_start[e] <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    m0 = (tile - g.tile_start[e]) * PF_BM;
    const int cnt = g.offsets[e + 1] - g.offsets[e];
    M = min(PF_BM, cnt - m0);
    pos0 = g.offsets[e] + m0;
  } else {
    m0 = blockIdx.x * PF_BM;
    if (m0 >= g.M_total) return;
    M = min(PF_BM, g.M_total - m0);
    pos0 = m0;
  }
  const int n0 = blockIdx.y * G_BN;
  const uint8_t* w = g.w + (size_t)e * g.w_stride;
  const uint16_t* wsc = g.ws ? g.ws + (size_t)e * g.ws_stride : nullptr;
  // A row index (into g.a) for each tile row
  if (tid < PF_BM) {
    int r = -1;
    if (tid < M) {
      const int pos = pos0 + tid;
      if (KIND == GK_GATE_UP && g.perm) r = g.perm[pos] / g.k;
      else r = pos;
    }
    s_row[tid] = r;
  }
  __syncthreads();

  const int nsub = (M + 15) >> 4;  // active 16-row subtiles (wave-uniform)
  floatx4_t acc[G_MSUB][4];
#pragma unroll
  for (int i = 0; i < G_MSUB; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // loaders: A: thread -> (row tid/2, 16 elements at 16*(tid&1)); B: thread -> weight row n0 + tid
  const int arow = tid >> 1, ahalf = tid & 1;
  const int asrc = s_row[arow];
  const int bn = n0 + tid;
  const int nsteps = g.K / G_BK;
  uint4 ra0 = make_uint4(0, 0, 0, 0), ra1 = make_uint4(0, 0, 0, 0);
  uint32_t rb[32];
  float rs = 0.0f;
  auto load_step = [&](int s) {
    if (asrc >= 0) {
      const uint4* src = reinterpret_cast<const uint4*>(g.a + (size_t)asrc * g.K + s * G_BK + 16 * ahalf);
      ra0 = src[0];
      ra1 = src[1];
    }
    if (bn < g.N) load_b_chunk<WT>(g, w, wsc, bn, s, rb, rs);
  };
  load_step(0);
  for (int s = 0; s < nsteps; s++) {
    // stage step s into LDS
    {
      uint4* da = reinterpret_cast<uint4*>(sA + arow * G_LDA + 16 * ahalf);
      da[0] = ra0;
      da[1] = ra1;
      uint32_t bq[16];
      if (bn < g.N) {
        dequant_b_chunk<WT>(rb, rs, bq);
      } else {
#pragma unroll
        for (int i = 0; i < 16; i++) bq[i] = 0;
      }
      uint4* db = reinterpret_cast<uint4*>(sB + tid * G_LDA);
#pragma unroll
      for (int i = 0; i < 4; i++) db[i] = make_uint4(bq[4 * i], bq[4 * i + 1], bq[4 * i + 2], bq[4 * i + 3]);
    }
    __syncthreads();
    if (s + 1 < nsteps) load_step(s + 1);
    // MFMA: wave owns weight-row subtiles 4*wave .. 4*wave+3
    bf16x8_t bfrag[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = (4 * wave + j) * 16 + (lane & 15);
      bfrag[j] = *reinterpret_cast<const bf16x8_t*>(sB + col * G_LDA + 8 * (lane >> 4));
    }
#pragma unroll
    for (int i = 0; i < G_MSUB; i++) {
      if (i < nsub) {
        const int row = 16 * i + (lane & 15);
        const bf16x8_t afrag = *reinterpret_cast<const bf16x8_t*>(sA + row * G_LDA + 8 * (lane >> 4));
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // ---- epilogue. acc[i][j] lane l: weight row (4*wave + j)*16 + (l & 15) of the tile,
  //      token rows 16 i + 4 (l >> 4) + r
  if (KIND == GK_GATE_UP) {
    // subtiles (4w, 4w+1) = gate/up rows of group 2w of the tile, (4w+2, 4w+3) = group 2w+1
    const int I = g.N / 2;
#pragma unroll
    for (int i = 0; i < G_MSUB; i++) {
      if (i < nsub) {
#pragma unroll
        for (int gg = 0; gg < 2; gg++) {
          const int col = (n0 / 32 + 2 * wave + gg) * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int m = 16 * i + 4 * (lane >> 4) + r;
            if (m < M && col < I) {
              const float gv = acc[i][2 * gg][r], uv = acc[i][2 * gg + 1][r];
              g.out[(size_t)(pos0 + m) * I + col] = f32_to_bf16(silu_f32(gv) * uv);
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < G_MSUB; i++) {
      if (i < nsub) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int col = n0 + (4 * wave + j) * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int m = 16 * i + 4 * (lane >> 4) + r;
            if (m < M && col < g.N) g.out[(size_t)(pos0 + m) * g.N + col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j g[t][j] Y[inv[t*k+j]] + Ys[t]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_combine(const uint16_t* __restrict__ Y, const uint16_t* __restrict__ Ys,
                                                     const int32_t* __restrict__ inv, const float* __restrict__ gates,
                                                     int T, int H, int k, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;
    for (int j = 0; j < k; j++) {
      const float gj = gates[(size_t)t * k + j];
      const uint4 v = *reinterpret_cast<const uint4*>(Y + (size_t)inv[(size_t)t * k + j] * H + c);
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] = __builtin_fmaf(gj, bf16_lo(vv[i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(gj, bf16_hi(vv[i]), acc[2 * i + 1]);
      }
    }
    if (Ys) {
      const uint4 v = *reinterpret_cast<const uint4*>(Ys + (size_t)t * H + c);
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] += bf16_lo(vv[i]);
        acc[2 * i + 1] += bf16_hi(vv[i]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + (size_t)t * H + c) = o;
  }
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
static hipError_t route_steps(const LayerDev& L, const uint16_t* x, int T, int32_t* idx_out, float* gate_out,
                              int32_t* counts_out, const PrefillWs& ws, hipStream_t st, bool permute) {
  const int E = L.E, k = L.k, H = L.H;
  (void)launch_k(KC_PF_ROUTER, k_pf_router, dim3((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N), dim3(256), 0, st, L.router_w,
                     L.router_b, x, T, E, H, ws.logits);
  (void)launch_k(KC_PF_TOPK, k_pf_topk, dim3((T + 3) / 4), dim3(256), 0, st, ws.logits, T, E, k, ws.idx, ws.gates, idx_out,
                     gate_out);
  if (!permute && !counts_out) return hipGetLastError();
  const int nblk = (T + PF_TOK_PER_BLK - 1) / PF_TOK_PER_BLK;
  (void)launch_k(KC_PF_COUNT, k_pf_count, dim3(nblk), dim3(256), E * sizeof(int), st, ws.idx, T, E, k, ws.blk_counts);
  (void)launch_k(KC_PF_SCAN, k_pf_scan, dim3(1), dim3(1024), 0, st, ws.blk_counts, nblk, E, ws.blk_base, ws.counts,
                     ws.offsets, ws.tile_start, counts_out);
  if (!permute) return hipGetLastError();
  (void)launch_k(KC_PF_SCATTER, k_pf_scatter, dim3(nblk), dim3(256), E * sizeof(int), st, ws.idx, T, E, k, ws.blk_base, ws.perm,
                     ws.inv);
  return hipGetLastError();
}

hipError_t launch_route(const LayerDev& L, const uint16_t* x, int T, int32_t* idx_out, float* gate_out,
                        int32_t* counts_out, const PrefillWs& ws, hipStream_t st) {
  return route_steps(L, x, T, idx_out, gate_out, counts_out, ws, st, false);
}

template <int WT, int KIND>
static void gemm_launch(int kc, const GemmArgs& g, int tiles_x, hipStream_t st) {
  (void)launch_k(kc, k_pf_gemm<WT, KIND>, dim3(tiles_x, (g.N + G_BN - 1) / G_BN), dim3(G_THREADS), 0, st, g);
}

template <int KIND>
static void gemm_dispatch(int kc, int wt, const GemmArgs& g, int tiles_x, hipStream_t st) {
  switch (wt) {
    case MOE_W_Q4: gemm_launch<MOE_W_Q4, KIND>(kc, g, tiles_x, st); break;
    case MOE_W_Q3: gemm_launch<MOE_W_Q3, KIND>(kc, g, tiles_x, st); break;
    case MOE_W_BF16: gemm_launch<MOE_W_BF16, KIND>(kc, g, tiles_x, st); break;
    default: gemm_launch<MOE_W_F32, KIND>(kc, g, tiles_x, st); break;
  }
}

hipError_t launch_prefill(const LayerDev& L, const uint16_t* x, int T, uint16_t* y, int32_t* idx_out, float* gate_out,
                          const PrefillWs& ws, hipStream_t st) {
  const int E = L.E, k = L.k, H = L.H, I = L.I;
  hipError_t err = route_steps(L, x, T, idx_out, gate_out, nullptr, ws, st, true);
  if (err != hipSuccess) return err;
  const int max_tiles = (T * k + PF_BM - 1) / PF_BM + E;
  const bool quant = (L.wt == MOE_W_Q4 || L.wt == MOE_W_Q3);
  // routed gate/up
  {
    GemmArgs g{};
    g.w = L.gu; g.ws = quant ? L.gu_s : nullptr; g.w_stride = L.gu_stride; g.ws_stride = L.gu_s_stride;
    g.N = 2 * I; g.K = H; g.a = x; g.perm = ws.perm; g.k = k;
    g.offsets = ws.offsets; g.tile_start = ws.tile_start; g.E = E; g.out = ws.h;
    gemm_dispatch<GK_GATE_UP>(KC_PF_GATE_UP, L.wt, g, max_tiles, st);
  }
  // shared gate/up
  if (L.swt != MOE_W_NONE) {
    GemmArgs g{};
    g.w = L.sgu; g.N = 2 * I; g.K = H; g.a = x; g.perm = nullptr; g.k = k;
    g.offsets = nullptr; g.M_total = T; g.out = ws.hs;
    gemm_dispatch<GK_GATE_UP>(KC_PF_SHARED_GATE_UP, L.swt, g, (T + PF_BM - 1) / PF_BM, st);
  }
  // routed down
  {
    GemmArgs g{};
    g.w = L.dn; g.ws = quant ? L.dn_s : nullptr; g.w_stride = L.dn_stride; g.ws_stride = L.dn_s_stride;
    g.N = H; g.K = I; g.a = ws.h; g.perm = nullptr; g.k = k;
    g.offsets = ws.offsets; g.tile_start = ws.tile_start; g.E = E; g.out = ws.Y;
    gemm_dispatch<GK_DOWN>(KC_PF_DOWN, L.wt, g, max_tiles, st);
  }
  if (L.swt != MOE_W_NONE) {
    GemmArgs g{};
    g.w = L.sdn; g.N = H; g.K = I; g.a = ws.hs; g.perm = nullptr; g.k = k;
    g.offsets = nullptr; g.M_total = T; g.out = ws.Ys;
    gemm_dispatch<GK_DOWN>(KC_PF_SHARED_DOWN, L.swt, g, (T + PF_BM - 1) / PF_BM, st);
  }
  (void)launch_k(KC_PF_COMBINE, k_pf_combine, dim3(T), dim3(256), 0, st, ws.Y, (L.swt != MOE_W_NONE) ? ws.Ys : nullptr, ws.inv,
                     ws.gates, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
