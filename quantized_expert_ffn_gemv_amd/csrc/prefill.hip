// Prefill path: T tokens through one MoE layer.
//
//   k_pf_rsplit      router weights -> two bf16 halves and row norms
//   k_pf_rapprox     approximate router logits, bf16 MFMA (error bounded)
//   k_pf_rselect     per token: candidates from the bounds, their exact fp64
//                    logits, ordered top-k and renormalised gates
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
// Router: logits[t][e] = sum_h W[e][h] x[t][h] + b[e] in fp64, then the
// ordered top-k. Selection needs the exact fp64 order only near the k-th
// largest logit, so the logits are filtered first and verified after:
//   k_pf_rsplit   W (fp32) -> W_hi = bf16(W), W_lo = bf16(W - W_hi) and
//                 ||W_e||_2 in fp64 (|W - W_hi - W_lo| <= 2^-16 |W|);
//   k_pf_gemm<bf16, GK_F32> (the dense grouped GEMM, one "expert" of 2E
//                 rows) computes W_hi x and W_lo x with bf16 MFMA, fp32
//                 sums; a[t][e] = (W_hi x + W_lo x) + b in fp32;
//   k_pf_rselect  per token: |a - l| <= B_e = C ||W_e|| ||x_t|| + 2^-22 |a|
//                 + 2^-100 (below); L = the k-th largest a - B; candidates =
//                 experts with a + B >= L (every top-k expert is one: k
//                 experts have l >= L, and a + B < L means l < L); their
//                 exact fp64 logits (fp32 weight x bf16 activation is exact
//                 in fp64, sums in fp64), ordered top-k among them (value,
//                 then lower index), renormalised gates.
// The bound: the split leaves 2^-16 S (S = sum |W x| <= ||W|| ||x||); each
// accumulator sums 2048-ish exact products (bf16 x bf16 fits fp32) in fp32,
// error <= gamma_n S with gamma_n = n u / (1 - n u), taken with u = 2^-23
// (directed rounding) and n = H + 32 (the MFMA's own partial sums); the
// final adds cost 2^-23 (|a| + |b|) each. C covers all of it with a factor > 1.1
// spare; 2^-110 ||x|| + 2^-100 absorb flushed denormal weights and sums.
// ---------------------------------------------------------------------------
// The halves land as one chunk-major bf16 matrix of 2E rows (hi rows, then lo
// rows; chunk c of row r = elements 8c .. 8c+7 at [c][r]), the layout the
// dense grouped GEMM reads.
__global__ __launch_bounds__(256) void k_pf_rsplit(const float* __restrict__ W, int E, int H, uint16_t* __restrict__ split,
                                                   double* __restrict__ wnorm) {
  // one workgroup per expert row; thread: chunks c = threadIdx.x + 256 j
  __shared__ double s_ss[4];
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* w = W + (size_t)e * H;
  double ss = 0.0;
  for (int c = threadIdx.x; c < (H >> 3); c += 256) {
    const float4 v0 = *reinterpret_cast<const float4*>(w + 8 * c);
    const float4 v1 = *reinterpret_cast<const float4*>(w + 8 * c + 4);
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      ph[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
      pl[q] = pack_bf16x2(f[2 * q] - bf16_lo(ph[q]), f[2 * q + 1] - bf16_hi(ph[q]));
    }
    *reinterpret_cast<uint4*>(split + ((size_t)c * 2 * E + e) * 8) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    *reinterpret_cast<uint4*>(split + ((size_t)c * 2 * E + E + e) * 8) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
    for (int q = 0; q < 8; q++) ss = __builtin_fma((double)f[q], (double)f[q], ss);
  }
  ss = wave_total_f64(ss);
  if (lane == 0) s_ss[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) wnorm[e] = __builtin_sqrt((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]));
}

// One wave per token (E <= 1024: lane holds experts lane + 64 i); approx is
// [T][2E]: the W_hi x and W_lo x sums. The
// token's activations stay in registers (NXH chunks of 512: lane holds
// hidden 512 j + 8 lane .. + 7); candidates go four at a time (their weight
// rows load together), each exact logit summed across the wave in a fixed
// order (DPP rows, then the four row sums).
constexpr int RS_NV = 16;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int NXH, bool SPLIT>
__global__ __launch_bounds__(256) void k_pf_rselect(const float* __restrict__ W, const float* __restrict__ bias,
                                                    const uint16_t* __restrict__ x, const float* __restrict__ approx,
                                                    const float* __restrict__ approx2,
                                                    const double* __restrict__ wnorm, int T, int E, int H, int k,
                                                    int32_t* __restrict__ idx, float* __restrict__ gates,
                                                    int32_t* idx_out, float* gate_out) {
  __shared__ int s_ce[4][64 * RS_NV];     // candidate experts, ascending
  __shared__ uint32_t s_key[4][64];       // lane maxima of the lower ends (sortable keys)
  __shared__ double s_ov[4][16];          // winners in order
  __shared__ int s_oe[4][16];
  __shared__ double s_cv[4][64 * RS_NV];  // exact logits of the candidates, in candidate order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave; no workgroup barrier below
  int* cl = s_ce[wave];
  const uint16_t* xt = x + (size_t)t * H;
  // activations and ||x_t||_2 (fp64)
  // (held in registers for H <= 2048; longer rows are reloaded per chunk, an
  // L1 hit, instead of living in an array the compiler would put in memory)
  constexpr bool XR = NXH <= 4;
  auto x_chunk = [&](int j) {
    const int h = 512 * j + 8 * lane;
    const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xt + min(h, H - 8)));
    return (h < H) ? make_uint4(vv.x, vv.y, vv.z, vv.w) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xr[XR ? NXH : 1];
  double xs = 0.0;
#pragma unroll
  for (int j = 0; j < NXH; j++) {
    const uint4 v = x_chunk(j);
    if constexpr (XR) xr[j] = v;
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const double a = bf16_lo(p[q]), b = bf16_hi(p[q]);
      xs = __builtin_fma(a, a, xs);
      xs = __builtin_fma(b, b, xs);
    }
  }
  const double xn = __builtin_sqrt(wave_total_f64(xs));
  // bounds; lower ends a_e - B_e, upper ends a_e + B_e
  const double C = (1.1 * ((double)(H + 32) * 0x1p-23 / (1.0 - (double)(H + 32) * 0x1p-23)) + 0x1p-15) * (1.0 + 1e-9);
  double lo[RS_NV], up[RS_NV];
#pragma unroll
  for (int i = 0; i < RS_NV; i++) {
    const int e = lane + 64 * i;
    const int ec = min(e, E - 1);
    const float bv = bias ? bias[ec] : 0.0f;
    // (the approximate logits and x are read once: non-temporal, so that
    // they do not push the router rows out of the L2)
    // (split K: each half's two parts added first; the bound below covers
    // any summation order of the H products in fp32)
    float ahi = __builtin_nontemporal_load(approx + (size_t)t * 2 * E + ec);
    float alo = __builtin_nontemporal_load(approx + (size_t)t * 2 * E + E + ec);
    if constexpr (SPLIT) {
      ahi += __builtin_nontemporal_load(approx2 + (size_t)t * 2 * E + ec);
      alo += __builtin_nontemporal_load(approx2 + (size_t)t * 2 * E + E + ec);
    }
    const double a = (double)((ahi + alo) + bv);
    const double B = C * wnorm[ec] * xn + 0x1p-22 * (__builtin_fabs(a) + __builtin_fabs((double)bv)) + 0x1p-110 * xn + 0x1p-100;
    lo[i] = (e < E) ? a - B : -__builtin_inf();
    up[i] = (e < E) ? a + B : -__builtin_inf();
  }
  // L = a lower bound of the k-th largest lower end: the k-th largest of the
  // lanes' maxima (k lanes hold a lower end >= it), by the leading 26 bits
  // of its sortable key (ties between lanes broken by lane, so the 64 keys
  // are distinct); L = the smallest fp64 value with those leading bits.
  double lmax = -__builtin_inf();
#pragma unroll
  for (int i = 0; i < RS_NV; i++) lmax = lo[i] > lmax ? lo[i] : lmax;
  const uint32_t key = (sort_key_hi(lmax) & ~63u) | (uint32_t)(63 - lane);
  s_key[wave][lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rk0 = 0, rk1 = 0;
  const uint4* kv = reinterpret_cast<const uint4*>(s_key[wave]);
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const uint4 q = kv[j], q2 = kv[j + 1];
    rk0 += (int)(q.x > key) + (int)(q.y > key) + (int)(q.z > key) + (int)(q.w > key);
    rk1 += (int)(q2.x > key) + (int)(q2.y > key) + (int)(q2.z > key) + (int)(q2.w > key);
  }
  const uint64_t selk = __ballot(rk0 + rk1 == k - 1);
  const double L = key_floor_value((uint32_t)__builtin_amdgcn_readlane((int)key, __ffsll((long long)selk) - 1) & ~63u);
  // candidates, in expert order
  int nc = 0;
#pragma unroll
  for (int i = 0; i < RS_NV; i++) {
    const bool c = up[i] >= L;
    const uint64_t bal = __ballot(c);
    if (c) cl[nc + __popcll(bal & ((1ull << lane) - 1ull))] = lane + 64 * i;
    nc += __popcll(bal);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // exact logits, four candidates per pass (each written to LDS by one lane)
  double* cvl = s_cv[wave];
  for (int c0 = 0; c0 < nc; c0 += 4) {
    int e[4];
    double acc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      e[q] = cl[min(c0 + q, nc - 1)];
      acc[q] = 0.0;
    }
    constexpr int UJ = NXH <= 4 ? NXH : 2;  // weight loads in flight per pass
#pragma unroll UJ
    for (int j = 0; j < NXH; j++) {
      const int h = min(512 * j + 8 * lane, H - 8);  // lanes past H: x is zero there
      float4 w[4][2];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float* we = W + (size_t)e[q] * H + h;
        w[q][0] = *reinterpret_cast<const float4*>(we);
        w[q][1] = *reinterpret_cast<const float4*>(we + 4);
      }
      double xj[8];
      uint4 xv;
      if constexpr (XR) xv = xr[j];
      else xv = x_chunk(j);
      const uint32_t p[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int r = 0; r < 4; r++) {
        xj[2 * r] = bf16_lo(p[r]);
        xj[2 * r + 1] = bf16_hi(p[r]);
      }
#pragma unroll
      for (int q = 0; q < 4; q++) {
        acc[q] = __builtin_fma((double)w[q][0].x, xj[0], acc[q]);
        acc[q] = __builtin_fma((double)w[q][0].y, xj[1], acc[q]);
        acc[q] = __builtin_fma((double)w[q][0].z, xj[2], acc[q]);
        acc[q] = __builtin_fma((double)w[q][0].w, xj[3], acc[q]);
        acc[q] = __builtin_fma((double)w[q][1].x, xj[4], acc[q]);
        acc[q] = __builtin_fma((double)w[q][1].y, xj[5], acc[q]);
        acc[q] = __builtin_fma((double)w[q][1].z, xj[6], acc[q]);
        acc[q] = __builtin_fma((double)w[q][1].w, xj[7], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const double l = wave_total_f64(acc[q]) + (bias ? (double)bias[e[q]] : 0.0);
      if (lane == q && c0 + q < nc) cvl[c0 + q] = l;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // candidate c in lane c % 64, slot c / 64
  double cv[RS_NV];
#pragma unroll
  for (int i = 0; i < RS_NV; i++) {
    const int c = lane + 64 * i;
    cv[i] = (c < nc) ? cvl[min(c, 64 * RS_NV - 1)] : -__builtin_inf();
  }
  // ordered top-k among the candidates (value, then lower expert index)
  if (nc <= 64) {
    // rank of candidate c (lane c) by counting the candidates before it
    const double myc = cv[0];
    const int mye = cl[min(lane, nc - 1)];
    int rk = 0;
    for (int j = 0; j < nc; j++) {
      const double vj = readlane_f64(myc, j);
      const int ej = __builtin_amdgcn_readlane(mye, j);
      rk += (int)((vj > myc) | ((vj == myc) & (ej < mye)));
    }
    if (lane < nc && rk < k) {
      s_ov[wave][rk] = myc;
      s_oe[wave][rk] = mye;
    }
  } else {
    int ce[RS_NV];
#pragma unroll
    for (int i = 0; i < RS_NV; i++) {
      const int c = lane + 64 * i;
      ce[i] = (c < nc) ? cl[min(c, nc - 1)] : 0x7FFFFFFF;
    }
    for (int r = 0; r < k; r++) {
      double best = -__builtin_inf();
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < RS_NV; i++)
        if (cv[i] > best || (cv[i] == best && ce[i] < bi)) { best = cv[i]; bi = ce[i]; }
      wave_argmax(best, bi);
#pragma unroll
      for (int i = 0; i < RS_NV; i++)
        if (ce[i] == bi) cv[i] = -__builtin_inf(), ce[i] = 0x7FFFFFFF;
      if (lane == 0) {
        s_ov[wave][r] = best;
        s_oe[wave][r] = bi;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // renormalised gates: softmax of the k selected fp64 logits
  const double m = s_ov[wave][0];
  const double myv = s_ov[wave][lane < k ? lane : 0];
  const int myi = s_oe[wave][lane < k ? lane : 0];
  const double ev = (lane < k) ? exp(myv - m) : 0.0;
  const double z = wave_total_f64(ev);
  if (lane < k) {
    const float g = (float)(ev / z);
    const int ix = (myi >= 0 && myi < E) ? myi : 0;  // in range whatever the inputs held
    idx[(size_t)t * k + lane] = ix;
    gates[(size_t)t * k + lane] = g;
    if (idx_out) idx_out[(size_t)t * k + lane] = ix;
    if (gate_out) gate_out[(size_t)t * k + lane] = g;
  }
}

// ---------------------------------------------------------------------------
// Histogram / scan / stable permutation
// ---------------------------------------------------------------------------
constexpr int PF_HT = 1024;  // threads of the histogram and permutation kernels (one block of tokens each)
__global__ __launch_bounds__(PF_HT) void k_pf_count(const int32_t* __restrict__ idx, int T, int E, int k,
                                                     int32_t* __restrict__ blk_counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += PF_HT) hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * PF_TOK_PER_BLK;
  const int t1 = min(T, t0 + PF_TOK_PER_BLK);
  // all of the thread's slots loaded first (clamped, unconditional), then counted
  constexpr int NPASS = PF_TOK_PER_BLK * 16 / PF_HT;  // k <= 16
  const int s0 = t0 * k, s1 = t1 * k;
  int ev[NPASS];
#pragma unroll
  for (int q = 0; q < NPASS; q++) ev[q] = idx[min(s0 + PF_HT * q + (int)threadIdx.x, s1 - 1)];
#pragma unroll
  for (int q = 0; q < NPASS; q++)
    if (s0 + PF_HT * q + (int)threadIdx.x < s1) atomicAdd(&hist[ev[q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PF_HT) blk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_pf_scan(const int32_t* __restrict__ blk_counts, int nblk, int E,
                                                   int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ tile_start,
                                                   int32_t* __restrict__ tile_info, int32_t* counts_out) {
  __shared__ int s_tot[1024];
  __shared__ int s_til[1024];
  const int e = threadIdx.x;
  // the expert's block counts, 32 loads in flight at a time (clamped,
  // unconditional; one round trip per 32 blocks instead of one per block)
  constexpr int SB = 32;
  const int ec = min(e, E - 1);
  int tot = 0;
  for (int b0 = 0; b0 < nblk; b0 += SB) {
    int v[SB];
#pragma unroll
    for (int j = 0; j < SB; j++) v[j] = blk_counts[(size_t)min(b0 + j, nblk - 1) * E + ec];
#pragma unroll
    for (int j = 0; j < SB; j++) tot += (b0 + j < nblk) ? v[j] : 0;
  }
  if (e >= E) tot = 0;
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
    const int ntiles = (tot + PF_BM - 1) / PF_BM;
    const int ts = s_til[e] - ntiles;
    tile_start[e] = ts;
    // per M tile: its expert and the expert's tile range and rows, so a GEMM
    // workgroup finds its tile with one lookup
    for (int t = 0; t < ntiles; t++) {
      int32_t* ti = tile_info + (size_t)PF_TILE_INFO * (ts + t);
      ti[0] = e; ti[1] = ts; ti[2] = ntiles; ti[3] = off; ti[4] = tot;
    }
    if (counts_out) counts_out[e] = tot;
    int run = off;
    for (int b0 = 0; b0 < nblk; b0 += SB) {
      int v[SB];
#pragma unroll
      for (int j = 0; j < SB; j++) v[j] = blk_counts[(size_t)min(b0 + j, nblk - 1) * E + e];
#pragma unroll
      for (int j = 0; j < SB; j++) {
        if (b0 + j < nblk) {
          blk_base[(size_t)(b0 + j) * E + e] = run;
          run += v[j];
        }
      }
    }
    if (e == E - 1) {
      offsets[E] = s_tot[e];
      tile_start[E] = s_til[e];
    }
  }
}

// Positions of the slots of one token block, in slot order within each expert.
// Per pass of PF_HT slots: each wave groups its lanes by expert (ballots),
// each group's leader posts the group's size for its wave, and a slot's
// position is the expert's running count + the sizes posted by the earlier
// waves + its rank in its group; then the running counts advance. (With 256
// threads a block of 256 tokens took ten such passes at top-10, 13.7 us for
// 4096 tokens on 16 workgroups.)
__global__ __launch_bounds__(PF_HT) void k_pf_scatter(const int32_t* __restrict__ idx, int T, int E, int k,
                                                       const int32_t* __restrict__ blk_base, int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv) {
  constexpr int NW = PF_HT / 64;
  extern __shared__ int cnt[];  // [E] running counts, then [NW][E] per-wave group sizes (bytes: at most 64)
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(cnt + E);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += PF_HT) {
    cnt[e] = blk_base[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < NW; w++) wcnt[w * E + e] = 0;
  }
  __syncthreads();
  const int t0 = blockIdx.x * PF_TOK_PER_BLK;
  const int t1 = min(T, t0 + PF_TOK_PER_BLK);
  const int s0 = t0 * k, s1 = t1 * k;
  int ebits = 0;
  while ((1 << ebits) < E) ebits++;
  // every pass's expert index loaded up front (clamped, unconditional): one
  // round trip for the block instead of one per pass; the pass loop is
  // unrolled so the values stay in registers
  constexpr int NPASS = PF_TOK_PER_BLK * 16 / PF_HT;  // k <= 16
  int ev[NPASS];
#pragma unroll
  for (int q = 0; q < NPASS; q++) ev[q] = idx[min(s0 + PF_HT * q + (int)threadIdx.x, s1 - 1)];
#pragma unroll
  for (int q = 0; q < NPASS; q++) {
    const int base = s0 + PF_HT * q;
    if (base >= s1) break;  // uniform
    const int s = base + threadIdx.x;
    const bool act = s < s1;
    const int e = act ? ev[q] : 0;
    // lanes of this wave with the same expert
    uint64_t peers = __ballot(act);
    for (int b = 0; b < ebits; b++) {
      const uint64_t m = __ballot(act && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    if (!act) peers = 0;
    const int before = __popcll(peers & ((1ull << lane) - 1ull));
    const bool leader = act && before == 0;
    if (leader) wcnt[wave * E + e] = (uint8_t)__popcll(peers);
    __syncthreads();
    if (act) {
      int pos = cnt[e] + before;
      // earlier waves' slots come first (all NW sizes read at once, masked)
#pragma unroll
      for (int w = 0; w < NW; w++) pos += (w < wave) ? (int)wcnt[w * E + e] : 0;
      perm[pos] = s;
      inv[s] = pos;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&cnt[e], __popcll(peers));
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM (MFMA 16x16x32 bf16, fp32 accumulate)
// ---------------------------------------------------------------------------
constexpr int G_THREADS = 256;     // 4 waves; wave w owns columns [16 NSW w, 16 NSW (w + 1)) of the tile
constexpr int G_BK = 128;          // K per pipeline stage (4 MFMA K-steps of 32)
constexpr int G_MSUB = PF_BM / 16; // 16-row subtiles per tile

enum GemmKind { GK_GATE_UP = 0, GK_DOWN = 1, GK_F32 = 2 };  // GK_F32: plain product, fp32 out (dense weights)

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
  const int32_t* tile_info;   // [tiles][PF_TILE_INFO]: expert, its first tile, its tiles, its row offset, its rows
  int E;
  int M_total;            // rows when offsets == NULL
  uint16_t* out;          // gate/up: h [rows][N/2]; down: Y [rows][N]
  float* out_f32;         // GK_F32: [rows][N]
  // GK_F32 over one matrix only: K split into ksplit equal parts, part p
  // written to out_f32 + p * out_plane (the caller adds the parts)
  int ksplit;
  ptrdiff_t out_plane;
};

// ---------------------------------------------------------------------------
// Weight fragments straight from HBM to registers. In one stage (K = 128,
// four 32-element blocks) lane l of a wave serves weight row n = l % 16 of a
// 16-column subtile and K block j = l / 16: it loads the whole block (one
// quantised chunk: 16 B Q4, 12 B Q3, plus its fp16 scale; 64 B bf16; 128 B
// fp32) and feeds MFMA step t = 0..3 with elements 8t .. 8t+7 of it. The
// MFMA therefore sees, for its k-group j, the actual K positions
// 32 j + 8 t + 0..7; the A fragments use the same positions, so the sum over
// K is unchanged. Lanes of consecutive rows read consecutive chunks of one
// chunk column (16 rows x 16 B = 256 contiguous bytes).
// ---------------------------------------------------------------------------
template <int WT> struct BRaw;
template <> struct BRaw<MOE_W_Q4> { uint4 w; uint32_t s; };          // s: fp16 scale bits, 0 when out of range
template <> struct BRaw<MOE_W_Q3> { uint32_t w0, w1, w2, s; };
template <> struct BRaw<MOE_W_BF16> { uint4 w[4]; uint32_t ok; };
template <> struct BRaw<MOE_W_F32> { uint4 w[8]; uint32_t ok; };

// Loads are unconditional (indices clamped into the matrix) so that no branch
// forces the compiler to wait for them; out-of-range blocks are zeroed when
// used (a zero scale for quantised types, a zero mask for dense ones).
// `cell` = (block, row) index blk * N + n of this lane's 32-element block,
// clamped into the matrix; `ok` = whether the unclamped block exists.
template <int WT>
__device__ __forceinline__ void load_b(const uint8_t* __restrict__ w, const uint16_t* __restrict__ ws, uint32_t N,
                                       uint32_t cell, bool ok, BRaw<WT>& r) {
  if constexpr (WT == MOE_W_Q4) {
    r.w = *reinterpret_cast<const uint4*>(w + cell * 16u);
    r.s = ws[cell] & (ok ? 0xFFFFu : 0u);
  } else if constexpr (WT == MOE_W_Q3) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(w + cell * 12u);
    r.w0 = p[0];
    r.w1 = p[1];
    r.w2 = p[2];
    r.s = ws[cell] & (ok ? 0xFFFFu : 0u);
  } else {
    // dense: the block is NCH consecutive 16-byte chunks of chunk columns NCH*blk .. ; cell -> (blk, n)
    constexpr uint32_t NCH = (WT == MOE_W_BF16) ? 4 : 8;
    const uint32_t blk = cell / N, n = cell - blk * N;
#pragma unroll
    for (uint32_t c = 0; c < NCH; c++) r.w[c] = *reinterpret_cast<const uint4*>(w + ((NCH * blk + c) * N + n) * 16u);
    r.ok = ok ? 0xFFFFFFFFu : 0u;
  }
}

// Elements 8t .. 8t+7 of the block as 4 bf16 pairs (the MFMA B fragment).
// Quantised: fp16(1024 + code) by a magic exponent, then s * (code - off)
// exactly in fp32 (one fma), rounded once to bf16.
template <int WT>
__device__ __forceinline__ bf16x8_t frag_b(const BRaw<WT>& r, int t) {
  uint32_t o[4];
  if constexpr (WT == MOE_W_Q4 || WT == MOE_W_Q3) {
    uint32_t p[4];
    if constexpr (WT == MOE_W_Q4) {
      const uint32_t wd = (t == 0) ? r.w.x : (t == 1) ? r.w.y : (t == 2) ? r.w.z : r.w.w;
      q4_word_pairs<F16_MAGIC2>(wd, p);
    } else {
      q3_group_pairs<F16_MAGIC2>(r.w0, r.w1, r.w2, t, p);
    }
    const float sc = f16_to_f32((uint16_t)r.s);
    const float negbase = -(1024.0f + (float)QOff<WT>::v) * sc;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float lo, hi;
      f16pair_dequant(p[i], sc, negbase, lo, hi);
      o[i] = pack_bf16x2(lo, hi);
    }
  } else if constexpr (WT == MOE_W_BF16) {
    const uint4 v = r.w[t];
    o[0] = v.x & r.ok; o[1] = v.y & r.ok; o[2] = v.z & r.ok; o[3] = v.w & r.ok;
  } else {
    const uint4 v0 = r.w[2 * t], v1 = r.w[2 * t + 1];
    o[0] = pack_bf16x2(__uint_as_float(v0.x), __uint_as_float(v0.y)) & r.ok;
    o[1] = pack_bf16x2(__uint_as_float(v0.z), __uint_as_float(v0.w)) & r.ok;
    o[2] = pack_bf16x2(__uint_as_float(v1.x), __uint_as_float(v1.y)) & r.ok;
    o[3] = pack_bf16x2(__uint_as_float(v1.z), __uint_as_float(v1.w)) & r.ok;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// ---------------------------------------------------------------------------
// Grouped GEMM. Tile = (M tile of one expert's rows, 256 weight rows).
// Workgroups go round-robin over the 8 XCDs; a contiguous range of logical
// tiles runs on each XCD. Routed: the tiles of one expert are consecutive,
// so the expert's weights and gathered rows stay in that XCD's L2 while they
// run; gate/up takes them M tile outer (an M tile's 4 KB rows are read once
// from memory for all its N tiles, the expert's 1 MB of weights stays in L2),
// down N tile outer (its rows are short, 1 KB; each weight tile is read
// once). One matrix for all tokens (shared expert, router): M tile outer,
// so the x rows are read from memory once rather than once per N tile.
//
// Pipeline, per 128-wide K stage: A (bf16 rows, gathered) goes straight from
// memory to LDS (global_load_lds, 16 B per lane) into a 2-slot ring; the
// weights go to registers one stage at a time; two waves per SIMD overlap one
// wave's loads and dequantisation with the other's MFMAs. One barrier per
// stage. The ring slots are separate LDS arrays and the loop is unrolled by
// 2, so each LDS read names its slot and the compiler need not wait for loads
// still in flight into the other slot.
// A rows in LDS: 16 chunks of 16 B per row, chunk c at position c ^ (row & 15)
// (conflict-free fragment reads without padding).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) const void* gbl_void_t;

constexpr int G_AROWS = PF_BM;                       // rows per A slot
constexpr int G_ALOADS = G_AROWS * 16 / G_THREADS;   // 16-byte DMA loads per lane per stage
constexpr int G_SLOT_U4 = G_AROWS * 16;              // uint4 per A slot

// 16-column weight subtiles per wave: 4 for quantised weights (16 B + a scale per
// lane and stage), 2 for dense ones (64 or 128 B per lane and stage)
template <int WT> constexpr int g_nsw() { return (WT == MOE_W_Q4 || WT == MOE_W_Q3) ? 4 : 2; }
template <int WT> constexpr int g_bn() { return 64 * g_nsw<WT>(); }
// vm operations per lane and stage for the weights (loads of all subtiles)
template <int WT> constexpr int b_vm_per_stage() {
  return g_nsw<WT>() * ((WT == MOE_W_Q4) ? 2 : (WT == MOE_W_Q3) ? 4 : (WT == MOE_W_BF16) ? 4 : 8);
}

template <int WT, int KIND>
__global__ __launch_bounds__(G_THREADS, 2) void k_pf_gemm(GemmArgs g) {
  __shared__ __align__(16) uint4 sA0[G_SLOT_U4];
  __shared__ __align__(16) uint4 sA1[G_SLOT_U4];
  __shared__ int s_row[PF_BM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-derived offsets live in SGPRs
  constexpr int NSW = g_nsw<WT>();
  constexpr int BN = g_bn<WT>();

  // ---- tile
  const int NT = (g.N + BN - 1) / BN;
  const int mt_total = g.offsets ? g.tile_start[g.E] : (g.M_total + PF_BM - 1) / PF_BM;
  const int nsplit = (KIND == GK_F32 && !g.offsets && g.ksplit > 1) ? g.ksplit : 1;
  const int total = mt_total * NT * nsplit;
  const int per = (total + 7) >> 3;
  const int ix = blockIdx.x >> 3;
  int logical = (blockIdx.x & 7) * per + ix;
  if (ix >= per || logical >= total) return;
  // K part of this tile (split K: the parts of one output tile are adjacent
  // in the list, so they run on one XCD and share its L2 copy of the rows)
  const int ksp = logical % nsplit;
  logical /= nsplit;
  const int Kp = g.K / nsplit, kofs = ksp * Kp;

  int e = 0, m0 = 0, M = 0, pos0 = 0, nt = 0;
  if (g.offsets) {
    const int32_t* ti = g.tile_info + (size_t)PF_TILE_INFO * (logical / NT);  // M tile q = logical / NT
    e = ti[0];
    const int ntiles = ti[2];
    const int pos = logical - NT * ti[1];
    nt = pos / ntiles;
    m0 = (pos - nt * ntiles) * PF_BM;
    M = min(PF_BM, ti[4] - m0);
    pos0 = ti[3] + m0;
  } else {
    const int mt = logical / NT;
    nt = logical - mt * NT;
    m0 = mt * PF_BM;
    M = min(PF_BM, g.M_total - m0);
    pos0 = m0;
  }
  const int n0 = nt * BN;
  const uint8_t* w = g.w + (size_t)e * g.w_stride;
  const uint16_t* wsc = g.ws ? g.ws + (size_t)e * g.ws_stride : nullptr;
  if (tid < PF_BM) {
    int r = 0;  // rows past M read row 0 of the matrix (finite values; their outputs are dropped)
    if (tid < M) {
      const int pos = pos0 + tid;
      r = (KIND == GK_GATE_UP && g.perm) ? g.perm[pos] / g.k : pos;
    }
    s_row[tid] = r;
  }
  __syncthreads();

  const int nsub = (M + 15) >> 4;  // active 16-row subtiles (uniform)
  floatx4_t acc[G_MSUB][NSW];
#pragma unroll
  for (int i = 0; i < G_MSUB; i++)
#pragma unroll
    for (int j = 0; j < NSW; j++) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nst = (Kp + G_BK - 1) / G_BK;
  // A DMA: wave w, load i covers slot rows 4 (G_ALOADS w + i) .. +3; lane -> row + lane / 16, position
  // lane % 16 holding chunk (lane % 16) ^ (row % 16)
  // The issue helpers derive their per-lane offsets from an opaque copy of the
  // lane index, so the compiler recomputes them (a few integer ops) at each
  // stage instead of keeping dozens of loop invariants live across the loop.
  auto issue_a = [&](int s, uint4* slot) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < G_ALOADS; i++) {
      const int row = 4 * (G_ALOADS * wave + i) + (ln >> 4);
      const int k = s * G_BK + 8 * ((ln & 15) ^ (row & 15));
      const uint16_t* src = g.a + (size_t)s_row[row] * g.K + kofs + (k < Kp ? k : 0);  // past K: a finite element (weight 0)
      __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(slot + 64 * (G_ALOADS * wave + i)), 16, 0, 0);
    }
  };
  // B: lane -> (row n = lane % 16 of each of the wave's 4 subtiles, K block j = lane / 16)
  const int bj = lane >> 4;
  const int nblk = Kp >> 5, blk0 = kofs >> 5;
  BRaw<WT> rb0[NSW];
  // lane's block of stage s: 4 s + bj; rows past N read row N - 1, blocks past K the stage's first block
  auto issue_b = [&](int s, BRaw<WT> (&r)[NSW]) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int j = ln >> 4;
    const bool okb = 4 * s + j < nblk;
    const uint32_t blk = (uint32_t)(blk0 + (okb ? 4 * s + j : 4 * s));
#pragma unroll
    for (int sub = 0; sub < NSW; sub++) {
      const int n = n0 + 16 * NSW * wave + (ln & 15) + 16 * sub;
      const bool ok = okb && n < g.N;
      const uint32_t cell = blk * (uint32_t)g.N + (uint32_t)(n < g.N ? n : g.N - 1);
      load_b<WT>(w, wsc, (uint32_t)g.N, cell, ok, r[sub]);
    }
  };
  // All G_MSUB row subtiles are computed (rows past M hold finite or stale
  // values whose results are never stored): no branch interrupts the MFMA
  // stream, and the A fragments of a step are read from LDS together.
  auto compute = [&](const uint4* A, const BRaw<WT> (&r)[NSW]) {
    const int m = lane & 15;
#pragma unroll
    for (int t = 0; t < 4; t++) {
      bf16x8_t bfrag[NSW];
#pragma unroll
      for (int sub = 0; sub < NSW; sub++) bfrag[sub] = frag_b<WT>(r[sub], t);
#pragma unroll
      for (int h = 0; h < G_MSUB; h += G_MSUB / 2) {  // row subtiles in two halves: fewer live fragments
        bf16x8_t afrag[G_MSUB / 2];
#pragma unroll
        for (int i = 0; i < G_MSUB / 2; i++)
          afrag[i] = __builtin_bit_cast(bf16x8_t, A[(16 * (h + i) + m) * 16 + ((4 * bj + t) ^ m)]);
#pragma unroll
        for (int i = 0; i < G_MSUB / 2; i++)
#pragma unroll
          for (int sub = 0; sub < NSW; sub++)
            acc[h + i][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[i], bfrag[sub], acc[h + i][sub], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // A: two-slot LDS ring; stage s + 1 is issued once every wave has passed
  // stage s's barrier (its slot, last read by stage s - 1, is then free) and
  // lands while stage s computes. Weights: one register stage, reloaded as
  // soon as a stage's MFMAs are issued; the second wave on each SIMD (another
  // workgroup) computes while this one waits for it.
  auto wait_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's loads of the stage have landed
    __builtin_amdgcn_s_barrier();        // ... and every other lane's
  };
  issue_a(0, sA0);
  issue_b(0, rb0);
  for (int s = 0; s < nst; s += 2) {
    wait_stage();
    if (s + 1 < nst) issue_a(s + 1, sA1);
    compute(sA0, rb0);
    if (s + 1 >= nst) break;
    issue_b(s + 1, rb0);
    wait_stage();
    if (s + 2 < nst) issue_a(s + 2, sA0);
    compute(sA1, rb0);
    if (s + 2 < nst) issue_b(s + 2, rb0);
  }

  // ---- epilogue. acc[i][j] lane l: weight row n0 + 16 NSW wave + 16 j + (l & 15),
  //      token rows 16 i + 4 (l >> 4) + r
  if (KIND == GK_GATE_UP) {
    // subtiles (2 gg, 2 gg + 1) = gate/up rows of interleave group n0/32 + (NSW/2) wave + gg
    const int I = g.N / 2;
#pragma unroll
    for (int i = 0; i < G_MSUB; i++) {
      if (i < nsub) {
#pragma unroll
        for (int gg = 0; gg < NSW / 2; gg++) {
          const int col = (n0 / 32 + (NSW / 2) * wave + gg) * 16 + (lane & 15);
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
        for (int j = 0; j < NSW; j++) {
          const int col = n0 + 16 * NSW * wave + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int m = 16 * i + 4 * (lane >> 4) + r;
            if (m < M && col < g.N) {
              if (KIND == GK_F32) g.out_f32[ksp * g.out_plane + (size_t)(pos0 + m) * g.N + col] = acc[i][j][r];
              else g.out[(size_t)(pos0 + m) * g.N + col] = f32_to_bf16(acc[i][j][r]);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM over quantised weights (Q4, Q3). Same tiles, A ring and
// fragment mapping as k_pf_gemm, but the weights also travel memory -> LDS by
// DMA, into a two-slot ring of per-wave regions (lane-private: 16 B per lane
// and subtile; Q3's three words in three 256-byte rows), so a whole stage of
// weights and A rows is in flight while the previous stage computes, with no
// weight registers held across it. LDS: 2 x 24 KB (A) + 2 x 16 KB (weights)
// = 80 KB per workgroup, two workgroups per CU; the gathered row of each of a
// lane's A loads is kept in a register instead of an LDS table.
//
// Q4 dequantisation, word t of a lane's block (elements 8t .. 8t+7: element
// 8t + 2p at nibble p, 8t + 2p + 1 at nibble p + 4): pairs 0 and 2 are masked
// to the low nibble of each half, fp16(1024 + code); pairs 1 and 3 keep their
// nibble in bits 4..7, fp16(1024 + 16 code). Both are exact in one fma each:
// s (code - 8) = fma(v, s, -1032 s) = fma(v, s / 16, -72 s) (every product
// and sum fits fp32), then one rounding to bf16.
// ---------------------------------------------------------------------------
struct Q4Scale { float s, s16, nb_even, nb_odd; };
__device__ __forceinline__ Q4Scale q4_scale(uint32_t sbits) {
  const float sc = f16_to_f32((uint16_t)sbits);
  return {sc, sc * 0.0625f, sc * -1032.0f, sc * -72.0f};
}
__device__ __forceinline__ bf16x8_t q4_frag(uint32_t wd, const Q4Scale& q, uint32_t magic) {
  const uint32_t w8 = wd >> 8;
  const uint32_t p[4] = {(wd & 0x000F000Fu) | magic, (wd & 0x00F000F0u) | magic,
                         (w8 & 0x000F000Fu) | magic, (w8 & 0x00F000F0u) | magic};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float lo, hi;
    if (i & 1) f16pair_dequant(p[i], q.s16, q.nb_odd, lo, hi);
    else f16pair_dequant(p[i], q.s, q.nb_even, lo, hi);
    o[i] = pack_bf16x2(lo, hi);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

constexpr int GQ_NSW = 4;                       // 16-column subtiles per wave
constexpr int GQ_BN = 64 * GQ_NSW;              // weight rows per tile
constexpr int GQ_REGION = 64 * 16;              // bytes per (wave, subtile) weight region
constexpr int GQ_BSLOT = (G_THREADS / 64) * GQ_NSW * GQ_REGION;  // 16 KB

// The tile's work with MSUB 16-row subtiles (2, 4, 5 or 6: the fewest that
// hold the tile's rows), so padding subtiles cost no MFMAs (an expert's last
// tile is often short; chosen per tile, so the loops stay branch-free).
template <int WT, int KIND, int MSUB>
__device__ __forceinline__ void gemm_q_tile(const GemmArgs& g, uint4* sA0, uint4* sA1, uint8_t* sB0, uint8_t* sB1, int e,
                                            int M, int pos0, int n0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NSW = GQ_NSW;
  const uint8_t* w = g.w + (size_t)e * g.w_stride;
  const uint16_t* wsc = g.ws + (size_t)e * g.ws_stride;

  // A rows of this lane's loads: load i covers slot rows 4 (G_ALOADS wave + i) + lane / 16
  // (rows past M read row 0 of the matrix: finite values whose results are dropped)
  // (loads unconditional with clamped indices: a load inside a branch makes
  // the compiler wait for it before going on, one round trip per row)
  uint32_t arow[G_ALOADS];
  int pv[G_ALOADS];
#pragma unroll
  for (int i = 0; i < G_ALOADS; i++) {
    const int row = 4 * (G_ALOADS * wave + i) + (lane >> 4);
    pv[i] = (KIND == GK_GATE_UP && g.perm) ? g.perm[pos0 + min(row, M - 1)] : 0;
  }
#pragma unroll
  for (int i = 0; i < G_ALOADS; i++) {
    const int row = 4 * (G_ALOADS * wave + i) + (lane >> 4);
    const int r = (KIND == GK_GATE_UP && g.perm) ? pv[i] / g.k : pos0 + row;
    arow[i] = (uint32_t)(row < M ? r : 0);
  }

  floatx4_t acc[MSUB][NSW];
#pragma unroll
  for (int i = 0; i < MSUB; i++)
#pragma unroll
    for (int j = 0; j < NSW; j++) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nst = (g.K + G_BK - 1) / G_BK;
  const int nblk = g.K >> 5;
  const int bj = lane >> 4;
  // fp16 scale bits of the lane's blocks and, beside them, which blocks are in
  // range (applied after the stage's wait: a use right after the load would
  // wait for every load in flight)
  uint32_t scl[2][NSW], okm[2];

  // one stage's loads into ring slot (sa, sb, scales sc, in-range bits ok)
  auto issue = [&](int s, uint4* sa, uint8_t* sb, uint32_t (&sc)[NSW], uint32_t& okbits) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recompute lane offsets per stage rather than hold them
#pragma unroll
    for (int i = 0; i < G_ALOADS; i++) {
      const int row = 4 * (G_ALOADS * wave + i) + (ln >> 4);
      const int k = s * G_BK + 8 * ((ln & 15) ^ (row & 15));
      const uint16_t* src = g.a + (size_t)arow[i] * g.K + (k < g.K ? k : 0);  // past K: finite (weight 0)
      __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(sa + 64 * (G_ALOADS * wave + i)), 16, 0, 0);
    }
    const int j = ln >> 4;
    const bool okb = 4 * s + j < nblk;  // blocks past K (also whole stages past the end): scale 0
    const uint32_t blk = (uint32_t)min(4 * s + j, nblk - 1);
    uint32_t bits = 0;
#pragma unroll
    for (int sub = 0; sub < NSW; sub++) {
      const int n = n0 + 16 * NSW * wave + (ln & 15) + 16 * sub;
      const bool ok = okb && n < g.N;
      const uint32_t cell = blk * (uint32_t)g.N + (uint32_t)(n < g.N ? n : g.N - 1);
      uint8_t* region = sb + (wave * NSW + sub) * GQ_REGION;
      if constexpr (WT == MOE_W_Q4) {
        __builtin_amdgcn_global_load_lds((gbl_void_t)(w + cell * 16u), (lds_void_t)region, 16, 0, 0);
      } else {
#pragma unroll
        for (int q = 0; q < 3; q++)
          __builtin_amdgcn_global_load_lds((gbl_void_t)(w + cell * 12u + 4u * q), (lds_void_t)(region + 256 * q), 4, 0, 0);
      }
      sc[sub] = wsc[cell];
      bits |= ok ? (1u << sub) : 0u;
    }
    okbits = bits;
  };

  uint32_t magic = F16_MAGIC2;
  asm volatile("" : "+v"(magic));  // held in a register: one and-or per pair
  const int m = lane & 15;
  auto compute = [&](const uint4* A, const uint8_t* sb, const uint32_t (&sc)[NSW], uint32_t okbits) {
    if constexpr (WT == MOE_W_Q4) {
      Q4Scale qs[NSW];
#pragma unroll
      for (int sub = 0; sub < NSW; sub++) qs[sub] = q4_scale(sc[sub] & ((okbits >> sub) & 1u ? 0xFFFFu : 0u));
      // each lane's 16-byte chunks in one 128-bit read per subtile (lanes
      // contiguous: no bank conflicts; four 32-bit reads at a 16-byte lane
      // stride put four lanes on every bank)
      uint4 wq[NSW];
#pragma unroll
      for (int sub = 0; sub < NSW; sub++) wq[sub] = reinterpret_cast<const uint4*>(sb + (wave * NSW + sub) * GQ_REGION)[lane];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        bf16x8_t bfrag[NSW];
#pragma unroll
        for (int sub = 0; sub < NSW; sub++) {
          const uint32_t wd = t == 0 ? wq[sub].x : t == 1 ? wq[sub].y : t == 2 ? wq[sub].z : wq[sub].w;
          bfrag[sub] = q4_frag(wd, qs[sub], magic);
        }
        {  // all row subtiles' A fragments of the step read together
          bf16x8_t afrag[MSUB];
#pragma unroll
          for (int i = 0; i < MSUB; i++)
            afrag[i] = __builtin_bit_cast(bf16x8_t, A[(16 * i + m) * 16 + ((4 * bj + t) ^ m)]);
#pragma unroll
          for (int i = 0; i < MSUB; i++)
#pragma unroll
            for (int sub = 0; sub < NSW; sub++)
              acc[i][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[i], bfrag[sub], acc[i][sub], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      BRaw<WT> r[NSW];
#pragma unroll
      for (int sub = 0; sub < NSW; sub++) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(sb + (wave * NSW + sub) * GQ_REGION) + lane;
        r[sub].w0 = p[0];
        r[sub].w1 = p[64];
        r[sub].w2 = p[128];
        r[sub].s = sc[sub] & ((okbits >> sub) & 1u ? 0xFFFFu : 0u);
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        bf16x8_t bfrag[NSW];
#pragma unroll
        for (int sub = 0; sub < NSW; sub++) bfrag[sub] = frag_b<WT>(r[sub], t);
        {  // all row subtiles' A fragments of the step read together
          bf16x8_t afrag[MSUB];
#pragma unroll
          for (int i = 0; i < MSUB; i++)
            afrag[i] = __builtin_bit_cast(bf16x8_t, A[(16 * i + m) * 16 + ((4 * bj + t) ^ m)]);
#pragma unroll
          for (int i = 0; i < MSUB; i++)
#pragma unroll
            for (int sub = 0; sub < NSW; sub++)
              acc[i][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[i], bfrag[sub], acc[i][sub], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  auto wait_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's loads of the stage have landed
    __builtin_amdgcn_s_barrier();        // ... and every other lane's
  };
  // Stage s + 1 is issued right after stage s's barrier: its A slot and this
  // wave's weight region were last read in stage s - 1, which every wave has
  // finished. The loop runs an even number of stages with no exit in between
  // (one exit keeps the accumulators in place): stages past the end load
  // in-range addresses with zero scales and add nothing; the wait after the
  // loop drains the last issue.
  const int nst2 = (nst + 1) & ~1;
  issue(0, sA0, sB0, scl[0], okm[0]);
  for (int s = 0; s < nst2; s += 2) {
    wait_stage();
    issue(s + 1, sA1, sB1, scl[1], okm[1]);
    compute(sA0, sB0, scl[0], okm[0]);
    wait_stage();
    issue(s + 2, sA0, sB0, scl[0], okm[0]);
    compute(sA1, sB1, scl[1], okm[1]);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- epilogue (as k_pf_gemm)
  const int nsub = (M + 15) >> 4;
  if (KIND == GK_GATE_UP) {
    const int I = g.N / 2;
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
      if (i < nsub) {
#pragma unroll
        for (int gg = 0; gg < NSW / 2; gg++) {
          const int col = (n0 / 32 + (NSW / 2) * wave + gg) * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int mm = 16 * i + 4 * (lane >> 4) + r;
            if (mm < M && col < I) {
              const float gv = acc[i][2 * gg][r], uv = acc[i][2 * gg + 1][r];
              g.out[(size_t)(pos0 + mm) * I + col] = f32_to_bf16(silu_f32(gv) * uv);
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
      if (i < nsub) {
#pragma unroll
        for (int j = 0; j < NSW; j++) {
          const int col = n0 + 16 * NSW * wave + 16 * j + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int mm = 16 * i + 4 * (lane >> 4) + r;
            if (mm < M && col < g.N) g.out[(size_t)(pos0 + mm) * g.N + col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

template <int WT, int KIND>
__global__ __launch_bounds__(G_THREADS, 2) void k_pf_gemm_q(GemmArgs g) {
  static_assert(WT == MOE_W_Q4 || WT == MOE_W_Q3, "quantised weights only");
  __shared__ __align__(16) uint4 sA0[G_SLOT_U4];
  __shared__ __align__(16) uint4 sA1[G_SLOT_U4];
  __shared__ __align__(16) uint8_t sB0[GQ_BSLOT];
  __shared__ __align__(16) uint8_t sB1[GQ_BSLOT];
  constexpr int BN = GQ_BN;

  // ---- tile (as k_pf_gemm)
  const int NT = (g.N + BN - 1) / BN;
  const int mt_total = g.offsets ? g.tile_start[g.E] : (g.M_total + PF_BM - 1) / PF_BM;
  const int total = mt_total * NT;
  const int per = (total + 7) >> 3;
  const int ix = blockIdx.x >> 3;
  const int logical = (blockIdx.x & 7) * per + ix;
  if (ix >= per || logical >= total) return;
  int e = 0, m0 = 0, M = 0, pos0 = 0, nt = 0;
  if (g.offsets) {
    const int32_t* ti = g.tile_info + (size_t)PF_TILE_INFO * (logical / NT);  // M tile q = logical / NT
    e = ti[0];
    const int ntiles = ti[2];
    const int pos = logical - NT * ti[1];
    if (KIND == GK_GATE_UP) {
      const int mt = pos / NT;
      nt = pos - mt * NT;
      m0 = mt * PF_BM;
    } else {
      nt = pos / ntiles;
      m0 = (pos - nt * ntiles) * PF_BM;
    }
    M = min(PF_BM, ti[4] - m0);
    pos0 = ti[3] + m0;
  } else {
    const int mt = logical / NT;
    nt = logical - mt * NT;
    m0 = mt * PF_BM;
    M = min(PF_BM, g.M_total - m0);
    pos0 = m0;
  }
  const int n0 = nt * BN;
  if (M <= 2 * 16) gemm_q_tile<WT, KIND, 2>(g, sA0, sA1, sB0, sB1, e, M, pos0, n0);
  else if (M <= 4 * 16) gemm_q_tile<WT, KIND, 4>(g, sA0, sA1, sB0, sB1, e, M, pos0, n0);
  else if (M <= 5 * 16) gemm_q_tile<WT, KIND, 5>(g, sA0, sA1, sB0, sB1, e, M, pos0, n0);
  else gemm_q_tile<WT, KIND, 6>(g, sA0, sA1, sB0, sB1, e, M, pos0, n0);
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j g[t][j] Y[inv[t*k+j]] + Ys[t]
// ---------------------------------------------------------------------------
constexpr int PF_KMAX = 16;  // slots per token the combine takes (k <= 16)
__global__ __launch_bounds__(256) void k_pf_combine(const uint16_t* __restrict__ Y, const uint16_t* __restrict__ Ys,
                                                     const int32_t* __restrict__ inv, const float* __restrict__ gates,
                                                     int T, int H, int k, uint16_t* __restrict__ y) {
  // One workgroup per token. The token's k slot positions and gates first
  // (one load each, clamped and unconditional), then the k rows' 16-byte
  // pieces of every column group all in flight together: one memory round
  // trip for the indices and one for the rows, not two per slot. Y, Ys and
  // y are touched once: non-temporal loads and stores (at 32768 tokens the
  // 1.3 GB of Y otherwise churns the caches: 335 -> 278 us).
  const int t = blockIdx.x;
  int pos[PF_KMAX];
  float gv[PF_KMAX];
#pragma unroll
  for (int j = 0; j < PF_KMAX; j++) {
    const size_t sj = (size_t)t * k + min(j, k - 1);
    pos[j] = inv[sj];
    gv[j] = (j < k) ? gates[sj] : 0.0f;
  }
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    uint4 v[PF_KMAX];
#pragma unroll
    for (int j = 0; j < PF_KMAX; j++) {
      const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Y + (size_t)pos[j] * H + c));
      v[j] = make_uint4(q.x, q.y, q.z, q.w);
    }
    uint4 vs = make_uint4(0u, 0u, 0u, 0u);
    if (Ys) {
      const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Ys + (size_t)t * H + c));
      vs = make_uint4(q.x, q.y, q.z, q.w);
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;
    // fixed slot order j = 0 .. k-1; slots past k (a repeat of slot k - 1)
    // are zeroed, so they add exactly 0 whatever that row holds
#pragma unroll
    for (int j = 0; j < PF_KMAX; j++) {
      const uint32_t m = (j < k) ? 0xFFFFFFFFu : 0u;
      const uint32_t vv[4] = {v[j].x & m, v[j].y & m, v[j].z & m, v[j].w & m};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] = __builtin_fmaf(gv[j], bf16_lo(vv[i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(gv[j], bf16_hi(vv[i]), acc[2 * i + 1]);
      }
    }
    if (Ys) {
      const uint32_t ss[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] += bf16_lo(ss[i]);
        acc[2 * i + 1] += bf16_hi(ss[i]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    const u32x4_t oq = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(oq, reinterpret_cast<u32x4_t*>(y + (size_t)t * H + c));
  }
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------
template <int WT, int KIND>
static void gemm_launch(int kc, const GemmArgs& g, int tiles_x, hipStream_t st) {
  // tiles_x: an upper bound on the M tiles; the kernel reads the real count and
  // maps workgroups XCD-major, so the grid is a multiple of 8
  const int nt = (g.N + g_bn<WT>() - 1) / g_bn<WT>();
  const int total = tiles_x * nt;
  if constexpr (WT == MOE_W_Q4 || WT == MOE_W_Q3) {
    static_assert(GQ_BN == g_bn<WT>(), "tile width");
    (void)launch_k(kc, k_pf_gemm_q<WT, KIND>, dim3(8 * ((total + 7) / 8)), dim3(G_THREADS), 0, st, g);
  } else {
    (void)launch_k(kc, k_pf_gemm<WT, KIND>, dim3(8 * ((total + 7) / 8)), dim3(G_THREADS), 0, st, g);
  }
}

static hipError_t route_steps(const LayerDev& L, const uint16_t* x, int T, int32_t* idx_out, float* gate_out,
                              int32_t* counts_out, const PrefillWs& ws, hipStream_t st, bool permute) {
  const int E = L.E, k = L.k, H = L.H;
  float* approx = reinterpret_cast<float*>(ws.logits);  // [T][2E] fp32 in the [T][E] fp64 area
  // Few tokens leave most of the GPU idle in the approximate-logit GEMM (a
  // 4096-token call has 344 tiles for 768 workgroup slots, each tile a chain
  // of 16 dependent K stages): K is then split in two, the second half's
  // products going to a plane in the per-slot output area (free until the
  // down GEMM), and the select adds the halves.
  const int rtiles = (T + PF_BM - 1) / PF_BM * ((2 * E + g_bn<MOE_W_BF16>() - 1) / g_bn<MOE_W_BF16>());
  const bool rsplit2 = 2 * rtiles <= 3 * 256 && H % (2 * G_BK) == 0 && (size_t)k * H >= (size_t)4 * E;
  float* approx2 = reinterpret_cast<float*>(ws.Y);
  (void)launch_k(KC_PF_RSPLIT, k_pf_rsplit, dim3(E), dim3(256), 0, st, L.router_w, E, H, ws.rsplit, ws.wnorm);
  {
    GemmArgs g{};
    g.w = reinterpret_cast<const uint8_t*>(ws.rsplit); g.N = 2 * E; g.K = H; g.a = x; g.perm = nullptr; g.k = 1;
    g.offsets = nullptr; g.M_total = T; g.out_f32 = approx;
    g.ksplit = rsplit2 ? 2 : 1;
    g.out_plane = approx2 - approx;
    gemm_launch<MOE_W_BF16, GK_F32>(KC_PF_ROUTER, g, g.ksplit * ((T + PF_BM - 1) / PF_BM), st);
  }
  {
    const int nxh = (H + 511) / 512;
    if (rsplit2) {
      auto sel = nxh <= 1 ? k_pf_rselect<1, true> : nxh <= 2 ? k_pf_rselect<2, true> : nxh <= 4 ? k_pf_rselect<4, true>
               : nxh <= 8 ? k_pf_rselect<8, true> : k_pf_rselect<16, true>;
      (void)launch_k(KC_PF_TOPK, sel, dim3((T + 3) / 4), dim3(256), 0, st, L.router_w, L.router_b, x, approx, approx2,
                     ws.wnorm, T, E, H, k, ws.idx, ws.gates, idx_out, gate_out);
    } else {
      auto sel = nxh <= 1 ? k_pf_rselect<1, false> : nxh <= 2 ? k_pf_rselect<2, false> : nxh <= 4 ? k_pf_rselect<4, false>
               : nxh <= 8 ? k_pf_rselect<8, false> : k_pf_rselect<16, false>;
      (void)launch_k(KC_PF_TOPK, sel, dim3((T + 3) / 4), dim3(256), 0, st, L.router_w, L.router_b, x, approx, approx,
                     ws.wnorm, T, E, H, k, ws.idx, ws.gates, idx_out, gate_out);
    }
  }
  if (!permute && !counts_out) return hipGetLastError();
  const int nblk = (T + PF_TOK_PER_BLK - 1) / PF_TOK_PER_BLK;
  (void)launch_k(KC_PF_COUNT, k_pf_count, dim3(nblk), dim3(PF_HT), E * sizeof(int), st, ws.idx, T, E, k, ws.blk_counts);
  (void)launch_k(KC_PF_SCAN, k_pf_scan, dim3(1), dim3(1024), 0, st, ws.blk_counts, nblk, E, ws.blk_base, ws.counts,
                     ws.offsets, ws.tile_start, ws.tile_info, counts_out);
  if (!permute) return hipGetLastError();
  (void)launch_k(KC_PF_SCATTER, k_pf_scatter, dim3(nblk), dim3(PF_HT), E * sizeof(int) + (PF_HT / 64) * E, st, ws.idx, T,
                 E, k, ws.blk_base, ws.perm,
                     ws.inv);
  return hipGetLastError();
}

hipError_t launch_route(const LayerDev& L, const uint16_t* x, int T, int32_t* idx_out, float* gate_out,
                        int32_t* counts_out, const PrefillWs& ws, hipStream_t st) {
  return route_steps(L, x, T, idx_out, gate_out, counts_out, ws, st, false);
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
    g.offsets = ws.offsets; g.tile_start = ws.tile_start; g.tile_info = ws.tile_info; g.E = E; g.out = ws.h;
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
    g.offsets = ws.offsets; g.tile_start = ws.tile_start; g.tile_info = ws.tile_info; g.E = E; g.out = ws.Y;
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
