// Batch-1 decode of one MoE layer as a single kernel.
//
// Workgroups take roles by index:
//
//   [0, nR)        router: 8 expert rows each, fp64 logits (an fp32 weight
//                  times a bf16 activation is exact in fp64).
//   [nR, +nSG)     shared expert: 8 intermediates each (16 gate/up rows),
//                  gate/up GEMV + SwiGLU -> h (bf16).        waits: logits
//                  (only so the router's bytes reach the chip first; the
//                  shared bytes then fill the memory-idle top-k window)
//   [.., +nRG)     routed experts: (slot, 16 intermediates) each; ordered
//                  top-k from the logits, then fused dequantise-GEMV of the
//                  32 gate/up rows + SwiGLU -> h (bf16).    waits: logits
//   down blocks    F_RD output rows each: top-k, then all down weights of
//                  its rows (k routed experts and the shared one) are loaded
//                  while the gate/up roles run; y = sum_i g_i D_i h_i +
//                  D_s h_s in a fixed order.          waits: logits, then h
//                  Block d runs on workgroup d once its router or shared
//                  role is done (extra workgroups after the routed ones take
//                  blocks beyond nR + nSG), so the whole grid fits on the
//                  chip at once.
//
// Progress: the routed gate/up workgroups wait only on the router, which
// never waits, so they always finish; a down block waits on them, and
// can only hold a slot they need if nR + nSG workgroups filled every slot
// on the chip, which 256 CUs rule out.
//
// Hand-off without cache flushes. Every value one workgroup passes to
// another (logits, h) travels in a 64-bit word whose high half is a tag
// that is new for every call (the call's epoch + 1), written and read with
// agent-scope relaxed atomics: each word is single-copy atomic and coherent
// across the chip's L2 slices on its own, and a reader uses a word only once
// its tag is current, so no release/acquire fence (an L2 write-back or
// invalidate per workgroup) is needed. Per-role counters are hints that
// keep polling traffic low: one thread per workgroup spins on the counter,
// then the words are read and checked. Every spin is bounded; one that runs
// out sets an error bit in the workspace and lets the workgroup finish, so
// the kernel always ends. The last workgroup to finish resets the counters
// and advances the epoch, so the workspace is ready for the next call (and
// for graph replay) without a memset.
//
// No float atomics: each value has one writer and every sum has a fixed
// order, so results are bitwise reproducible.
#include "moe_device.h"
#include "moe_internal.h"
#include "dec_common.h"

namespace moe {

constexpr int F_THREADS = 512;
constexpr int F_RCPL = 8;                       // router float4 chunks per lane and batch
constexpr uint64_t F_WAIT_TICKS = 1ull << 25;   // ~0.34 s of the 100 MHz wall clock

// Workspace sync area (uint32 words; every counter in its own 128-byte line).
// The logits and h counters and the epoch have one replica per XCD, so the
// pollers of one XCD share a line of their own; producers bump every replica.
constexpr int SY_LINE = 32;                                   // words per line
constexpr int SY_NREP = 8;                                    // replicas (XCDs)
constexpr int SY_LOGITS = 1 * SY_LINE;                        // + r * SY_LINE
constexpr int SY_H = (1 + SY_NREP) * SY_LINE;                 // + r * SY_LINE
constexpr int SY_EPOCH = (1 + 2 * SY_NREP) * SY_LINE;         // + r * SY_LINE
constexpr int SY_DONE = (1 + 3 * SY_NREP) * SY_LINE;
constexpr int SY_ERR = 0;
constexpr int SY_WORDS = (2 + 3 * SY_NREP) * SY_LINE;         // 3328 bytes
constexpr int F_SLOTS = 4;  // logits/h buffers rotate over this many calls

struct FusedGeo {
  int nR, nSG, nRG;  // router, shared gate/up, routed gate/up workgroups
  int nD;            // down blocks: block d < nR + nSG runs on workgroup d after its first role,
                     // the rest on extra workgroups after the routed ones
};

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ld_word_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_error(uint32_t* sync, uint32_t bit) {
  __hip_atomic_fetch_or(sync + SY_ERR, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int my_rep() { return blockIdx.x & (SY_NREP - 1); }

// Count the workgroup in on every replica once its tagged stores are issued.
// The count may become visible before the stores do; readers check tags.
__device__ __forceinline__ void count_in(uint32_t* sync, int which) {
  __syncthreads();
  if (threadIdx.x < SY_NREP)
    __hip_atomic_fetch_add(sync + which + SY_LINE * threadIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until this XCD's replica of counter `which` reaches target;
// the whole workgroup leaves together.
__device__ __forceinline__ void wait_hint(uint32_t* sync, int which, uint32_t target) {
  if (threadIdx.x == 0) {
    const uint32_t* c = sync + which + SY_LINE * my_rep();
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (ld_u32(c) < target) {
      __builtin_amdgcn_s_sleep(4);
      if ((++it & 15) == 0 && wall_clock64() - t0 > F_WAIT_TICKS) {
        flag_error(sync, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// A word loaded once: if its tag is not current yet (the producer's store
// is still on its way), reload it (bounded).
__device__ __forceinline__ uint64_t settle(const uint64_t* p, uint64_t w, uint32_t tag, uint32_t* sync) {
  if ((uint32_t)(w >> 32) != tag) {
    const uint64_t t0 = wall_clock64();
    w = ld_word_coherent(p);
    int it = 0;
    while ((uint32_t)(w >> 32) != tag) {
      __builtin_amdgcn_s_sleep(4);
      w = ld_word_coherent(p);
      if ((++it & 15) == 0 && wall_clock64() - t0 > F_WAIT_TICKS) {
        flag_error(sync, 2u);
        break;
      }
    }
  }
  return w;
}

__device__ __forceinline__ void finish(uint32_t* sync) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(sync + SY_DONE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {  // every other workgroup is past all of its waits
      const uint32_t next = ld_u32(sync + SY_EPOCH) + 1u;
      for (int r = 0; r < SY_NREP; r++) {
        __hip_atomic_store(sync + SY_LOGITS + SY_LINE * r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sync + SY_H + SY_LINE * r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sync + SY_EPOCH + SY_LINE * r, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(sync + SY_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Router: wave w of workgroup b computes the logit of expert 8b + w.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void role_router(const LayerDev& L, const uint16_t* __restrict__ x, uint64_t* logits, int b,
                                            uint32_t tag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = b * 8 + wave;
  const bool valid = e < L.E;
  const int n4 = L.H >> 2;
  const float4* wr = reinterpret_cast<const float4*>(L.router_w + (size_t)(valid ? e : 0) * L.H);
  const uint2* xv = reinterpret_cast<const uint2*>(x);
  double a0 = 0.0, a1 = 0.0;
  for (int c0 = 0; c0 < n4; c0 += 64 * F_RCPL) {
    float4 w[F_RCPL];
    uint2 xx[F_RCPL];
#pragma unroll
    for (int i = 0; i < F_RCPL; i++) {
      const int c = c0 + lane + 64 * i;
      const bool in = valid && c < n4;
      w[i] = in ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      xx[i] = in ? xv[c] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < F_RCPL; i++) {
      a0 = __builtin_fma((double)w[i].x, (double)bf16_lo(xx[i].x), a0);
      a1 = __builtin_fma((double)w[i].y, (double)bf16_hi(xx[i].x), a1);
      a0 = __builtin_fma((double)w[i].z, (double)bf16_lo(xx[i].y), a0);
      a1 = __builtin_fma((double)w[i].w, (double)bf16_hi(xx[i].y), a1);
    }
  }
  const double tot = wave_total_f64(a0 + a1);
  if (valid && lane == 0) {
    const uint64_t v = (uint64_t)__double_as_longlong(tot + (L.router_b ? (double)L.router_b[e] : 0.0));
    // two words (low, high half of the fp64 logit), each with the tag
    st_word(logits + 2 * e, (uint32_t)v, tag);
    st_word(logits + 2 * e + 1, (uint32_t)(v >> 32), tag);
  }
}

// ---------------------------------------------------------------------------
// Gate/up rows of one expert: RPW rows per workgroup (32 = 16 gate + 16 up
// rows of one interleave group; 16 = half a group), SwiGLU, h -> hout.
// Lane -> (row rr = lane % RPW, k-part kp); lanes with consecutive rows read
// consecutive 16-byte chunks (rows are contiguous within a chunk column).
// ---------------------------------------------------------------------------
template <int WT> constexpr int gu_batch() { return is_q<WT>() ? 4 : 8; }

template <int WT, int RPW>
__device__ __forceinline__ void gate_up_rows(const uint8_t* __restrict__ gu, const uint16_t* __restrict__ gus, int H,
                                             int R, int q, int hf, const uint16_t* xs, const float* xsum, float* s_red,
                                             uint64_t* hout, uint32_t tag) {
  constexpr int KC = kchunk<WT>();
  constexpr int NKP = F_THREADS / RPW;  // k-parts
  constexpr int NB = gu_batch<WT>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane % RPW;
  const int kp = lane / RPW + (64 / RPW) * wave;
  const int row = (RPW == 32) ? 32 * q + rr : 32 * q + 8 * hf + (rr & 7) + ((rr >> 3) << 4);
  const int nc = H / KC;
  float acc = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += NKP * NB) {
    Raw raw[NB];
    float sc[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int c = c0 + kp + NKP * i;
      if (c < nc) {
        raw[i] = load_chunk<WT>(gu, (size_t)c * R + row);
        if constexpr (is_q<WT>()) sc[i] = f16_to_f32(gus[(size_t)c * R + row]);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int c = c0 + kp + NKP * i;
      if (c < nc) {
        if constexpr (is_q<WT>())
          acc = __builtin_fmaf(sc[i], qdot32<WT>(raw[i], xs + 32 * c, xsum[c]), acc);
        else
          acc = ddot<WT>(raw[i], xs + (size_t)c * KC, acc);
      }
    }
  }
  // lanes of one wave that share a row: fold them first (fixed order)
  if constexpr (RPW == 16) acc += __shfl_xor(acc, 16, 64);
  if constexpr (RPW <= 32) acc += __shfl_xor(acc, 32, 64);
  if (lane < RPW) s_red[wave * RPW + rr] = acc;
  __syncthreads();
  if ((int)threadIdx.x < RPW / 4) {  // two intermediates per thread, one tagged word
    const int j = 2 * threadIdx.x;
    float g0 = 0.0f, u0 = 0.0f, g1 = 0.0f, u1 = 0.0f;
#pragma unroll
    for (int w = 0; w < F_THREADS / 64; w++) {
      g0 += s_red[w * RPW + j];
      u0 += s_red[w * RPW + RPW / 2 + j];
      g1 += s_red[w * RPW + j + 1];
      u1 += s_red[w * RPW + RPW / 2 + j + 1];
    }
    st_word(hout + threadIdx.x, pack_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1), tag);
  }
  (void)NKP;
}

// x -> LDS (bf16) and, for quantised weights, its 32-element block sums.
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int H, uint16_t* xs, float* xsum) {
  const int n8 = H >> 3;  // 16-byte chunks
  for (int i = threadIdx.x; i < n8; i += F_THREADS) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    reinterpret_cast<uint4*>(xs)[i] = v;
    if (xsum) {
      float s = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
                ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
      s += dpp_f32<DPP_XOR1>(s);  // chunks 4b..4b+3 are lanes 4b'..4b'+3 of one quad
      s += dpp_f32<DPP_XOR2>(s);
      if ((i & 3) == 0) xsum[i >> 2] = s;
    }
  }
}

constexpr int F_NV = 8;  // logits per lane in the top-k: E <= 512 on this path

// Top-k of the token by wave 0 from the tagged logits; the workgroup reads
// idx/gates from LDS after.
__device__ __forceinline__ void block_topk(const uint64_t* logits, int E, int k, uint32_t tag, uint32_t* sync,
                                           uint8_t* scratch, int* s_idx, float* s_gate) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    uint64_t wl[F_NV], wh[F_NV];
#pragma unroll
    for (int i = 0; i < F_NV; i++) {
      const int e = lane + 64 * i;
      if (e < E) {  // coherent loads: a line another call left in this XCD's L2 is never used
        wl[i] = ld_word_coherent(logits + 2 * e);
        wh[i] = ld_word_coherent(logits + 2 * e + 1);
      }
    }
    double lv[F_NV];
#pragma unroll
    for (int i = 0; i < F_NV; i++) {
      const int e = lane + 64 * i;
      lv[i] = -__builtin_inf();
      if (e < E) {
        const uint64_t lo = settle(logits + 2 * e, wl[i], tag, sync);
        const uint64_t hi = settle(logits + 2 * e + 1, wh[i], tag, sync);
        lv[i] = __longlong_as_double((long long)(((hi & 0xFFFFFFFFull) << 32) | (lo & 0xFFFFFFFFull)));
      }
    }
    int mi;
    float mg;
    wave_topk(lv, E, k, lane, scratch, mi, mg);
    if (lane < k) {
      s_idx[lane] = mi;
      s_gate[lane] = mg;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Down role: output rows r0 .. r0 + F_RD - 1.
// Items: routed (j < k, block b < I/32, row rr) and shared (block b, row rr);
// an item is 32 consecutive columns of one row: one quantised chunk + scale,
// or 4 (bf16) / 8 (fp32) dense chunks.
// ---------------------------------------------------------------------------
template <int WT> constexpr int dn_batch() { return is_q<WT>() ? 6 : (WT == MOE_W_BF16 ? 2 : 1); }
template <int WT> constexpr int item_chunks() { return is_q<WT>() ? 1 : 32 / kchunk<WT>(); }

template <int WT>
struct Item {
  Raw r[item_chunks<WT>()];
  float s;
};

template <int WT>
__device__ __forceinline__ void load_item(const uint8_t* __restrict__ d, const uint16_t* __restrict__ ds, int H, int row,
                                          int b, Item<WT>& it) {
  constexpr int NCH = item_chunks<WT>();
#pragma unroll
  for (int c = 0; c < NCH; c++) it.r[c] = load_chunk<WT>(d, (size_t)(b * NCH + c) * H + row);
  if constexpr (is_q<WT>()) it.s = f16_to_f32(ds[(size_t)b * H + row]);
}

template <int WT>
__device__ __forceinline__ float item_dot(const Item<WT>& it, const uint16_t* h32, float hsum) {
  if constexpr (is_q<WT>()) {
    return it.s * qdot32<WT>(it.r[0], h32, hsum);
  } else {
    constexpr int NCH = item_chunks<WT>();
    constexpr int KC = kchunk<WT>();
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; c++) a = ddot<WT>(it.r[c], h32 + KC * c, a);
    return a;
  }
}

constexpr int F_RD = 16;  // output rows per down block

template <int WT, int SWT>
__device__ __forceinline__ void role_down(const LayerDev& L, const FusedGeo& G, const DecodeWs& ws, uint16_t* __restrict__ y,
                                          int d, uint8_t* smem, uint32_t tag, const uint64_t* tl, const uint64_t* th) {
  const int H = L.H, I = L.I, E = L.E, k = L.k;
  const int nB = I >> 5;
  constexpr bool HAS_S = SWT != MOE_W_NONE;
  constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
  const int r0 = d * F_RD;
  const int nj = k + (HAS_S ? 1 : 0);
  // LDS: h [nj][I] bf16 | hsum [k][nB] | part [nj][nB][F_RD] | pj [nj][F_RD] | idx, gate [16] | top-k scratch
  uint16_t* s_h = reinterpret_cast<uint16_t*>(smem);
  float* s_hsum = reinterpret_cast<float*>(smem + (((size_t)nj * I * 2 + 15) & ~(size_t)15));
  float* s_part = s_hsum + k * nB;
  float* s_pj = s_part + (size_t)nj * nB * F_RD;
  int* s_idx = reinterpret_cast<int*>(s_pj + nj * F_RD);
  float* s_gate = reinterpret_cast<float*>(s_idx + 16);
  uint8_t* s_tk = smem + ((reinterpret_cast<uint8_t*>(s_gate + 16) - smem + 15) & ~(ptrdiff_t)15);

  wait_hint(ws.sync, SY_LOGITS, (uint32_t)G.nR);
  // the top-k first: its logits loads must not queue behind weight loads
  block_topk(tl, E, k, tag, ws.sync, s_tk, s_idx, s_gate);
  // shared items
  const int nsi = nB * F_RD;
  Item<SW> si;
  const int st = threadIdx.x;
  if constexpr (HAS_S) {
    if (st < nsi) {
      const int row = r0 + st % F_RD;
      if (row < H) load_item<SW>(L.sdn, nullptr, H, row, st / F_RD, si);
    }
  }
  // routed items, first batch issued now
  constexpr int NB = dn_batch<WT>();
  const int nri = k * nB * F_RD;
  Item<WT> it[NB];
  auto issue = [&](int base) {
#pragma unroll
    for (int n = 0; n < NB; n++) {
      const int i = base + (int)threadIdx.x + F_THREADS * n;
      if (i < nri) {
        const int rr = i % F_RD, b = (i / F_RD) % nB, j = i / (F_RD * nB);
        const int row = r0 + rr;
        const int e = s_idx[j];
        if (row < H)
          load_item<WT>(L.dn + (size_t)e * L.dn_stride, is_q<WT>() ? L.dn_s + (size_t)e * L.dn_s_stride : nullptr, H,
                        row, b, it[n]);
      }
    }
  };
  issue(0);
  wait_hint(ws.sync, SY_H, (uint32_t)(G.nSG + G.nRG));
  // stage h (slot order, then shared) from its tagged words, and the routed block sums
  {
    const uint64_t* hw = th;
    const int nw = (nj * I) >> 1;
    constexpr int HB = 8;
    for (int w0 = 0; w0 < nw; w0 += F_THREADS * HB) {
      uint64_t v[HB];
#pragma unroll
      for (int n = 0; n < HB; n++) {
        const int w = w0 + (int)threadIdx.x + F_THREADS * n;
        if (w < nw) v[n] = ld_word_coherent(hw + w);
      }
#pragma unroll
      for (int n = 0; n < HB; n++) {
        const int w = w0 + (int)threadIdx.x + F_THREADS * n;
        if (w < nw) reinterpret_cast<uint32_t*>(s_h)[w] = (uint32_t)settle(hw + w, v[n], tag, ws.sync);
      }
    }
    __syncthreads();
    if constexpr (is_q<WT>()) {
      for (int i = threadIdx.x; i < k * nB; i += F_THREADS) {
        const uint4* v = reinterpret_cast<const uint4*>(s_h + (size_t)i * 32);
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const uint4 q = v[c];
          a += ((bf16_lo(q.x) + bf16_hi(q.x)) + (bf16_lo(q.y) + bf16_hi(q.y))) +
               ((bf16_lo(q.z) + bf16_hi(q.z)) + (bf16_lo(q.w) + bf16_hi(q.w)));
        }
        s_hsum[i] = a;
      }
      __syncthreads();
    }
  }
  // routed items
  for (int base = 0; base < nri; base += F_THREADS * NB) {
    if (base > 0) issue(base);
#pragma unroll
    for (int n = 0; n < NB; n++) {
      const int i = base + (int)threadIdx.x + F_THREADS * n;
      if (i < nri) {
        const int rr = i % F_RD, b = (i / F_RD) % nB, j = i / (F_RD * nB);
        const float hs = is_q<WT>() ? s_hsum[j * nB + b] : 0.0f;
        s_part[(size_t)(j * nB + b) * F_RD + rr] = (r0 + rr < H) ? item_dot<WT>(it[n], s_h + (size_t)j * I + 32 * b, hs) : 0.0f;
      }
    }
  }
  if constexpr (HAS_S) {
    if (st < nsi) {
      const int rr = st % F_RD, b = st / F_RD;
      s_part[(size_t)(k * nB + b) * F_RD + rr] = (r0 + rr < H) ? item_dot<SW>(si, s_h + (size_t)k * I + 32 * b, 0.0f) : 0.0f;
    }
  }
  __syncthreads();
  // per (expert, row): sum over blocks; then y = sum_j g_j s_j + s_shared
  for (int t = threadIdx.x; t < nj * F_RD; t += F_THREADS) {
    const int j = t / F_RD, rr = t % F_RD;
    const float* p = s_part + (size_t)j * nB * F_RD + rr;
    float a0 = 0.0f, a1 = 0.0f;
    int b = 0;
    for (; b + 1 < nB; b += 2) {
      a0 += p[b * F_RD];
      a1 += p[(b + 1) * F_RD];
    }
    if (b < nB) a0 += p[b * F_RD];
    s_pj[t] = a0 + a1;
  }
  __syncthreads();
  if ((int)threadIdx.x < F_RD) {
    const int rr = threadIdx.x;
    float acc = 0.0f;
    for (int j = 0; j < k; j++) acc = __builtin_fmaf(s_gate[j], s_pj[j * F_RD + rr], acc);
    if (HAS_S) acc += s_pj[k * F_RD + rr];
    if (r0 + rr < H) y[r0 + rr] = f32_to_bf16(acc);
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int WT, int SWT>
__global__ __launch_bounds__(F_THREADS) void k_decode1(LayerDev L, const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ y, int32_t* idx_out, float* gate_out,
                                                       DecodeWs ws, FusedGeo G) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_idx[16];
  __shared__ float s_gate[16];
  const int H = L.H, I = L.I;
  // this call's tag: the epoch (stable until every workgroup is done) + 1
  const uint32_t tag = ld_u32(ws.sync + SY_EPOCH + SY_LINE * my_rep()) + 1u;
  uint64_t* tl = reinterpret_cast<uint64_t*>(ws.logits) + (size_t)(tag % F_SLOTS) * 2 * L.E;
  uint64_t* th = reinterpret_cast<uint64_t*>(ws.h) + (size_t)(tag % F_SLOTS) * ((L.k + 1) * I / 2);
  int b = blockIdx.x;
  if (b < G.nR) {
    role_router(L, x, tl, b, tag);
    count_in(ws.sync, SY_LOGITS);
  } else if ((b -= G.nR) < G.nSG) {
    // shared expert, intermediates 16q + 8hf .. +7
    constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* s_red = reinterpret_cast<float*>(smem + (size_t)H * 2);
    stage_x(x, H, xs, nullptr);
    wait_hint(ws.sync, SY_LOGITS, (uint32_t)G.nR);  // the router's bytes first; these fill the top-k window
    const int q = b >> 1, hf = b & 1;
    gate_up_rows<SW, 16>(L.sgu, nullptr, H, 2 * I, q, hf, xs, nullptr, s_red,
                         th + (((size_t)L.k * I + 16 * q + 8 * hf) >> 1), tag);
    count_in(ws.sync, SY_H);
  } else if ((b -= G.nSG) < G.nRG) {
    // routed slot u, intermediates 16q .. 16q+15
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + (size_t)H * 2);
    float* s_red = reinterpret_cast<float*>(smem + (((size_t)H * 2 + (H >> 5) * 4 + 15) & ~(size_t)15));
    uint8_t* s_tk = reinterpret_cast<uint8_t*>(s_red + 8 * 32);
    stage_x(x, H, xs, is_q<WT>() ? xsum : nullptr);
    wait_hint(ws.sync, SY_LOGITS, (uint32_t)G.nR);
    block_topk(tl, L.E, L.k, tag, ws.sync, s_tk, s_idx, s_gate);
    const int gpe = I >> 4;
    const int u = b / gpe, q = b - u * gpe;
    if (b == 0 && (int)threadIdx.x < L.k) {
      if (idx_out) idx_out[threadIdx.x] = s_idx[threadIdx.x];
      if (gate_out) gate_out[threadIdx.x] = s_gate[threadIdx.x];
    }
    const int e = s_idx[u];
    gate_up_rows<WT, 32>(L.gu + (size_t)e * L.gu_stride, is_q<WT>() ? L.gu_s + (size_t)e * L.gu_s_stride : nullptr, H,
                         2 * I, q, 0, xs, xsum, s_red, th + (((size_t)u * I + 16 * q) >> 1), tag);
    count_in(ws.sync, SY_H);
  }
  // down blocks
  const int first = G.nR + G.nSG, extra0 = first + G.nRG;
  int d = -1;
  if ((int)blockIdx.x < first) d = blockIdx.x;
  else if ((int)blockIdx.x >= extra0) d = first + ((int)blockIdx.x - extra0);
  if (d >= 0 && d < G.nD) role_down<WT, SWT>(L, G, ws, y, d, smem, tag, tl, th);
  finish(ws.sync);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static size_t lds_gate_up(int H) {
  return (((size_t)H * 2 + (size_t)(H >> 5) * 4 + 15) & ~(size_t)15) + 8 * 32 * 4 + TOPK_SCRATCH;
}
static size_t lds_down(int I, int k, bool has_s) {
  const size_t nj = k + (has_s ? 1 : 0), nB = I >> 5;
  return (((size_t)nj * I * 2 + 15) & ~(size_t)15) + (((k * nB + nj * nB * F_RD + nj * F_RD + 32) * 4 + 15) & ~(size_t)15) +
         TOPK_SCRATCH;
}

size_t decode1_lds(int H, int I, int k, bool has_shared) {
  const size_t a = lds_gate_up(H), d = lds_down(I, k, has_shared);
  return a > d ? a : d;
}

bool decode1_fits(int E, int H, int I, int k, bool has_shared) {
  // F_NV logits per lane in the top-k, one shared-expert down item per thread
  // (I/32 * F_RD <= F_THREADS) and a 64 KiB LDS budget
  return E <= 64 * F_NV && I <= 1024 && decode1_lds(H, I, k, has_shared) <= 65536;
}

template <int WT, int SWT>
static hipError_t launch_fused_t(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out, float* gate_out,
                                 const DecodeWs& ws, hipStream_t st) {
  FusedGeo G;
  G.nR = (L.E + 7) / 8;
  G.nSG = (SWT == MOE_W_NONE) ? 0 : L.I / 8;
  G.nRG = L.k * (L.I / 16);
  G.nD = (L.H + F_RD - 1) / F_RD;
  const size_t lds = decode1_lds(L.H, L.I, L.k, SWT != MOE_W_NONE);
  const int extra = G.nD > G.nR + G.nSG ? G.nD - (G.nR + G.nSG) : 0;
  const int grid = G.nR + G.nSG + G.nRG + extra;
  return launch_k(KC_DEC_FUSED, k_decode1<WT, SWT>, dim3(grid), dim3(F_THREADS), lds, st, L, x, y, idx_out, gate_out,
                  ws, G);
}

template <int WT>
static hipError_t launch_fused_w(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* io, float* go,
                                 const DecodeWs& ws, hipStream_t st) {
  if (L.swt == MOE_W_NONE) return launch_fused_t<WT, MOE_W_NONE>(L, x, y, io, go, ws, st);
  if (L.swt == MOE_W_F32) return launch_fused_t<WT, MOE_W_F32>(L, x, y, io, go, ws, st);
  return launch_fused_t<WT, MOE_W_BF16>(L, x, y, io, go, ws, st);
}

hipError_t launch_decode_fused(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out, float* gate_out,
                               const DecodeWs& ws, hipStream_t st) {
  switch (L.wt) {
    case MOE_W_Q4: return launch_fused_w<MOE_W_Q4>(L, x, y, idx_out, gate_out, ws, st);
    case MOE_W_Q3: return launch_fused_w<MOE_W_Q3>(L, x, y, idx_out, gate_out, ws, st);
    case MOE_W_BF16: return launch_fused_w<MOE_W_BF16>(L, x, y, idx_out, gate_out, ws, st);
    default: return launch_fused_w<MOE_W_F32>(L, x, y, idx_out, gate_out, ws, st);
  }
}

}  // namespace moe
