// Batch-1 decode of one MoE layer as a single kernel.
//
// Workgroups take roles by index (nA = max(nR, nSG) first workgroups, then
// the routed ones, then extra reducers if needed; at most one workgroup per
// CU at the shapes of interest, so no role shares a CU's VALUs with another):
//
//   [0, nA)        b < nR: router, 8 expert rows each (two waves a row),
//                  fp64 logits (an fp32 weight times a bf16 activation is
//                  exact in fp64); then
//                  b < nSG: shared expert, 8 intermediates each (16 gate/up
//                  rows), gate/up GEMV + SwiGLU -> h (bf16, in LDS), then
//                  those 8 columns of the shared down matrix times h: a
//                  partial y over all H rows. The shared bytes stream while
//                  the routed workgroups wait for the logits and select.
//   [nA, +nRG)     routed experts: (slot, 32 intermediates) each; ordered
//                  top-k from the logits, then fused dequantise-GEMV of the
//                  64 gate/up rows + SwiGLU -> h (bf16, in LDS), then the
//                  matching 32-column block of the expert's down matrix
//                  (loaded with the gate/up rows) times h, scaled by the
//                  slot's gate: a partial y over all H rows. waits: logits
//   reducers       F_RD output rows each: y = the sum of the partials of
//                  all shared and routed roles in a fixed order. Reducers
//                  run on the last nD workgroups (routed ones after their
//                  own role; extra workgroups when nD > nRG).
//                                                waits: every partial
//
// The down product is split along the intermediate dimension (split-K), so
// h never leaves the workgroup that made it and the down weights stream
// together with the gate/up weights; the only hand-off after the top-k is
// the partials, read by the reducers.
//
// Progress: the routed workgroups wait only on the router roles, which
// never wait, and the shared roles never wait, so every partial gets
// written once every workgroup is resident; a reducer waits on producers
// dispatched after it, so the path is taken only when the whole grid fits
// on the chip at once (one workgroup per CU).
//
// Hand-off without cache flushes. Every value one workgroup passes to
// another (logits, partial down products) travels in a 64-bit word whose
// high half is a tag that is new for every call (the call's epoch + 1),
// written and read with agent-scope relaxed atomics: each word is
// single-copy atomic and coherent across the chip's L2 slices on its own,
// and a reader uses a word only once its tag is current, so no
// release/acquire fence (an L2 write-back or invalidate per workgroup) is
// needed. Each router role also writes one tagged flag word once its
// logits are issued; a routed workgroup polls those flags (one wave, one
// word per lane) and then reads and checks the logits; reducers poll the
// partial words directly. Flags are plain stores, one 128-byte line each:
// a shared counter bumped by hundreds of producers serialises its atomics
// at the memory side, and lines polled by hundreds of workgroups serve them
// one after another (both measured to add microseconds). Every spin is bounded;
// one that runs out sets an error bit in the workspace and lets the
// workgroup finish, so the kernel always ends. The last workgroup to finish
// (a per-XCD count, then a count of the XCD groups) resets the counts and
// advances the epoch, so the workspace is ready for the next call (and for
// graph replay) without a memset.
//
// No float atomics: each value has one writer and every sum has a fixed
// order, so results are bitwise reproducible.
#include "moe_device.h"
#include "moe_internal.h"
#include "dec_common.h"

namespace moe {

// 16 waves per workgroup, one workgroup per CU: four waves per SIMD keep
// the dequantise-dot chains busy (two waves per SIMD left the SIMDs idle
// through LDS and dependency latencies: the same work took 1.76x as long).
constexpr int F_THREADS = 1024;
constexpr int F_WAVES = F_THREADS / 64;
constexpr int F_RPT = 2;                        // down rows per thread (H <= F_RPT * F_THREADS)
constexpr int F_HMAX = F_RPT * F_THREADS;       // largest H of this path (LDS arrays are sized for it)
constexpr int F_RCPL = 4;                       // router float4 chunks per lane and batch
constexpr uint64_t F_WAIT_TICKS = 1ull << 25;   // ~0.34 s of the 100 MHz wall clock

// Workspace sync area (uint32 words; every count in its own 128-byte line).
// The epoch has one replica per XCD group (workgroups b with b % 8 == r), so
// the readers of one group share a line; one finish count for the grid.
constexpr int SY_LINE = 32;                                   // words per line
constexpr int SY_NREP = 8;                                    // replicas (XCD groups)
constexpr int SY_EPOCH = 1 * SY_LINE;                         // + r * SY_LINE
constexpr int SY_DONE = (1 + SY_NREP) * SY_LINE;
constexpr int SY_ERR = 0;
constexpr int SY_WORDS = (2 + SY_NREP) * SY_LINE;             // 1280 bytes
static_assert(SY_WORDS * 4 <= 4096, "sync area");
constexpr int F_SLOTS = 4;  // logits and flag buffers rotate over this many calls

struct FusedGeo {
  int nR, nSG, nRG;  // router, shared, routed roles
  int nA;            // workgroups [0, nA) take the router role (b < nR), then the shared role (b < nSG)
  int nD;            // reducers: reducer d < nA runs on workgroup d after its first roles,
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

// The workgroup's flag: written by one thread once every thread's tagged
// stores are issued (the flag may become visible before them; readers
// check the values' tags). Each flag has a 128-byte line of its own: with
// hundreds of workgroups polling, flags packed into a few lines made every
// poll queue behind the others at those lines (a hand-off took ~2 us
// instead of ~0.85 us, measured).
constexpr int F_FLAG_STRIDE = 16;  // uint64 words between flags
__device__ __forceinline__ void raise_flag(uint64_t* flags, int i, uint32_t tag) {
  __syncthreads();
  if (threadIdx.x == 0) st_word(flags + (size_t)F_FLAG_STRIDE * i, 0u, tag);
}

// Bounded wait until at least `need` of flags 0 .. n-1 carry the current tag
// (need <= n <= 64): wave 0 polls, one flag per lane per pass; the whole
// workgroup leaves together. Callers that pass need < n then read the
// values with per-word tag checks (settle), so the loads of the last
// producers' values overlap their arrival instead of following it.
__device__ __forceinline__ void wait_flags(const uint64_t* flags, int n, int need, uint32_t tag, uint32_t* sync) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      const uint64_t v = ld_word_coherent(flags + (size_t)F_FLAG_STRIDE * min(lane, n - 1));
      const int have = __popcll(__builtin_amdgcn_ballot_w64((lane < n) && (uint32_t)(v >> 32) == tag));
      if (have >= need) break;
      __builtin_amdgcn_s_sleep(1);
      if ((++it & 15) == 0 && wall_clock64() - t0 > F_WAIT_TICKS) {
        if (lane == 0) flag_error(sync, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// how many producer flags a consumer waits for before it reads the values
__device__ __forceinline__ int flags_needed(int n) { return n - n / 8; }

// A pair of words written together and loaded once: while either tag is
// not current (the producer's stores are still on their way), reload both
// (bounded).
__device__ __forceinline__ void settle2(const uint64_t* p0, const uint64_t* p1, uint64_t& w0, uint64_t& w1, uint32_t tag,
                                        uint32_t* sync) {
  if (((uint32_t)(w0 >> 32) != tag) | ((uint32_t)(w1 >> 32) != tag)) {
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(2);
      w0 = ld_word_coherent(p0);
      w1 = ld_word_coherent(p1);
      if (((uint32_t)(w0 >> 32) == tag) & ((uint32_t)(w1 >> 32) == tag)) break;
      if ((++it & 15) == 0 && wall_clock64() - t0 > F_WAIT_TICKS) {
        flag_error(sync, 2u);
        break;
      }
    }
  }
}

// Count the workgroup out; the last one (every other workgroup is past all
// of its waits) resets the count and advances the epoch for the next call.
// One count for the grid: its atomics are spread over the kernel's second
// half, and the last workgroup then waits one round trip, not two (a count
// per XCD group first, measured 0.09 us slower per call).
__device__ __forceinline__ void finish(uint32_t* sync) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(sync + SY_DONE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      const uint32_t next = ld_u32(sync + SY_EPOCH) + 1u;
      for (int q = 0; q < SY_NREP; q++)
        __hip_atomic_store(sync + SY_EPOCH + SY_LINE * q, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + SY_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Stack layers: z = RMSNorm(h) computed by every workgroup that reads the
// token, with the sum order of the library's RMSNorm kernel (threads
// 0..255 square and add 8 consecutive values each, each wave sums its lanes,
// then the four wave totals in order), so every workgroup and the separate
// kernel produce the same z. hv: the thread's 8 values of h (threads
// < H / 8; H <= F_HMAX = 256 x 8). Returns 1 / sqrt(mean(h^2) + eps) to every
// thread.
__device__ __forceinline__ float stack_inv(uint4 hv, int H, float eps, float* s_n) {
  float ss = 0.0f;
  if ((int)threadIdx.x * 8 < H) {
    const uint32_t vv[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = bf16_lo(vv[i]), b = bf16_hi(vv[i]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  if (threadIdx.x < 256) {
    ss = group_sum_f32(ss, 64);
    if ((threadIdx.x & 63) == 0) s_n[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  const float tot = s_n[0] + s_n[1] + s_n[2] + s_n[3];
  return 1.0f / sqrtf(tot / (float)H + eps);
}
__device__ __forceinline__ uint32_t scale_pair(uint32_t v, float inv) {
  return pack_bf16x2(bf16_lo(v) * inv, bf16_hi(v) * inv);
}

// ---------------------------------------------------------------------------
// Router: waves w and w + 8 of workgroup b compute the two halves of the
// logit of expert 8b + w (summed in that order). The
// logits are written once per XCD group (SY_NREP replicas): the routed
// workgroups of a group read their own copy, so each line has a few
// readers instead of all of them (lines read by hundreds of workgroups at
// once serve them one after another).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void role_router(const LayerDev& L, const uint16_t* __restrict__ x, uint64_t* logits, int b,
                                            double* s_rt, uint32_t tag, bool stk, float eps, float* s_n) {
  static_assert(F_WAVES == 16, "two waves per router row");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = b * 8 + (wave & 7), hh = wave >> 3;
  const bool valid = e < L.E;
  const int n4 = L.H >> 2, c_lo = hh * (n4 >> 1), c_hi = hh ? n4 : (n4 >> 1);
  const float4* wr = reinterpret_cast<const float4*>(L.router_w + (size_t)(valid ? e : 0) * L.H);
  const uint2* xv = reinterpret_cast<const uint2*>(x);
  // the bias is loaded with the weights (not after the sum: a load there is
  // one more memory round trip on the way to the top-k)
  const float* bp = L.router_b ? L.router_b + (valid ? e : 0) : L.router_w;
  const float bias_raw = *bp;
  double a0 = 0.0, a1 = 0.0;
  for (int c0 = c_lo; c0 < c_hi; c0 += 64 * F_RCPL) {
    float4 w[F_RCPL];
    uint2 xx[F_RCPL];
    // loads with clamped indices and no branch (a load inside a branch makes
    // the compiler wait for every load in flight where the branch joins);
    // elements past the row are masked after
#pragma unroll
    for (int i = 0; i < F_RCPL; i++) {
      const int c = min(c0 + lane + 64 * i, c_hi - 1);
      w[i] = wr[c];
      xx[i] = xv[c];
    }
    if (stk) {
      // stack layer: x is h, the activations are z = RMSNorm(h). Half a row
      // is one pass on this path (H <= F_HMAX), so the norm's loads go out
      // with the weights' and cost no round trip of their own.
      const uint4 hv = reinterpret_cast<const uint4*>(x)[min((int)threadIdx.x, (L.H >> 3) - 1)];
      const float inv = stack_inv(hv, L.H, eps, s_n);
#pragma unroll
      for (int i = 0; i < F_RCPL; i++) xx[i] = make_uint2(scale_pair(xx[i].x, inv), scale_pair(xx[i].y, inv));
    }
#pragma unroll
    for (int i = 0; i < F_RCPL; i++) {
      if (!(valid && c0 + lane + 64 * i < c_hi)) {
        w[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        xx[i] = make_uint2(0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < F_RCPL; i++) {
      a0 = __builtin_fma((double)w[i].x, (double)bf16_lo(xx[i].x), a0);
      a1 = __builtin_fma((double)w[i].y, (double)bf16_hi(xx[i].x), a1);
      a0 = __builtin_fma((double)w[i].z, (double)bf16_lo(xx[i].y), a0);
      a1 = __builtin_fma((double)w[i].w, (double)bf16_hi(xx[i].y), a1);
    }
  }
  const double part = wave_total_f64(a0 + a1);
  if (hh == 1 && lane == 0) s_rt[wave & 7] = part;
  __syncthreads();
  if (hh == 0 && valid && lane < SY_NREP) {
    const double tot = part + s_rt[wave];
    const uint64_t v = (uint64_t)__double_as_longlong(tot + (L.router_b ? (double)bias_raw : 0.0));
    // two words (low, high half of the fp64 logit), each with the tag, in
    // every XCD group's replica (lane r writes replica r)
    uint64_t* rl = logits + (size_t)lane * 2 * L.E;
    st_word(rl + 2 * e, (uint32_t)v, tag);
    st_word(rl + 2 * e + 1, (uint32_t)(v >> 32), tag);
  }
}

// qdot32 with the magic exponent held in a register: each code pair is one
// shift and one and-or (the constants then need no instruction of their own).
// The 32 bf16 activations come as four registers of eight (av).
template <int WT>
__device__ __forceinline__ float qdot32_regs(const Raw& r, const uint4 (&av)[4], float asum, uint32_t magic) {
  uint32_t p[16];
  if constexpr (WT == MOE_W_Q4) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int t = 0; t < 4; t++) p[4 * j + t] = ((r.w[j] >> (4 * t)) & 0x000F000Fu) | magic;
  } else {
    (void)magic;
    q3_pairs<BF16_MAGIC2>(r.w[0], r.w[1], r.w[2], p);
  }
  float c0 = -(128.0f + (float)QOff<WT>::v) * asum, c1 = 0.0f, c2 = 0.0f, c3 = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    c0 = dot2_bf16(p[4 * q + 0], av[q].x, c0);
    c1 = dot2_bf16(p[4 * q + 1], av[q].y, c1);
    c2 = dot2_bf16(p[4 * q + 2], av[q].z, c2);
    c3 = dot2_bf16(p[4 * q + 3], av[q].w, c3);
  }
  return (c0 + c1) + (c2 + c3);
}
template <int WT>
__device__ __forceinline__ float qdot32_reg(const Raw& r, const uint16_t* a, float asum, uint32_t magic) {
  const uint4* ap = reinterpret_cast<const uint4*>(a);
  const uint4 av[4] = {ap[0], ap[1], ap[2], ap[3]};
  return qdot32_regs<WT>(r, av, asum, magic);
}

// ---------------------------------------------------------------------------
// Gate/up rows of one expert -> SwiGLU -> h (bf16) in LDS.
//   RPW = 64: rows 64q .. 64q+63, two interleave groups of 32 rows (16 gate
//             rows, then their 16 up rows): intermediates 32q .. 32q+31;
//   RPW = 16: half a group, rows 32q + 8hf + (0..7) (gate) and + 16 (up):
//             intermediates 16q + 8hf .. +7.
// Lane -> (row rr = lane % RPW, k-part kp); lanes with consecutive rows read
// consecutive 16-byte chunks (rows are contiguous within a chunk column).
// Threads j < RPW/2 end holding intermediate j's value (returned, 0 for
// others), also stored to s_h[j].
// ---------------------------------------------------------------------------
constexpr int F_GU_NB = 4;  // chunks per thread and batch

template <int WT, int RPW, typename After>
__device__ __forceinline__ float gate_up_h(const uint8_t* __restrict__ gu, const uint16_t* __restrict__ gus, int H, int R,
                                           int q, int hf, const uint16_t* xs, const float* xsum, float* s_red,
                                           uint16_t* s_h, After&& after_first_issue) {
  constexpr int KC = kchunk<WT>();
  constexpr int NKP = F_THREADS / RPW;  // k-parts
  constexpr int NB = F_GU_NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane % RPW;
  const int kp = lane / RPW + (64 / RPW) * wave;
  const int row = (RPW == 64) ? 64 * q + rr : 32 * q + 8 * hf + (rr & 7) + ((rr >> 3) << 4);
  const int nc = H / KC;
  uint32_t magic = BF16_MAGIC2;
  asm volatile("" : "+v"(magic));  // a register operand: one and-or per code pair
  // batches known at compile time (H <= F_HMAX): straight-line code, so no
  // loop head makes the compiler wait for loads issued before it (the down
  // prefetch)
  constexpr int NBATCH = (F_HMAX / KC + NKP * NB - 1) / (NKP * NB);
  float acc = 0.0f;
#pragma unroll
  for (int bt = 0; bt < NBATCH; bt++) {
    const int c0 = bt * NKP * NB;
    Raw raw[NB];
    uint16_t sc[NB];  // fp16 bits: converted after the barrier, so no wait comes before it
    // clamped, unconditional loads (see role_router); each chunk's scale
    // right after it, so chunk i is computed as soon as its own two loads
    // are in (the waits count down in issue order) while later chunks
    // still stream
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const size_t o = (size_t)min(c0 + kp + NKP * i, nc - 1) * R + row;
      raw[i] = load_chunk<WT>(gu, o);
      if constexpr (is_q<WT>()) sc[i] = gus[o];
    }
    if (bt == 0) after_first_issue();  // loads needed later (the down columns) queue behind these
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before the first wait
    // every chunk is computed (no branch around the dot products): a chunk
    // past the row reads a valid chunk and contributes zero
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const bool in = c0 + kp + NKP * i < nc;
      const int c = min(c0 + kp + NKP * i, nc - 1);
      if constexpr (is_q<WT>()) {
        acc = __builtin_fmaf(in ? f16_to_f32(sc[i]) : 0.0f, qdot32_reg<WT>(raw[i], xs + 32 * c, xsum[c], magic), acc);
      } else {
        const float t = ddot<WT>(raw[i], xs + (size_t)c * KC, 0.0f);
        acc += in ? t : 0.0f;
      }
    }
  }
  // lanes of one wave that share a row: fold them first (fixed order)
  if constexpr (RPW == 16) acc += __shfl_xor(acc, 16, 64);
  if constexpr (RPW <= 32) acc += __shfl_xor(acc, 32, 64);
  if (lane < RPW) s_red[wave * RPW + rr] = acc;
  __syncthreads();
  float hv = 0.0f;
  if ((int)threadIdx.x < RPW / 2) {
    const int j = threadIdx.x;
    const int gi = (RPW == 16) ? j : 32 * (j >> 4) + (j & 15);
    const int ui = (RPW == 16) ? j + 8 : gi + 16;
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int w = 0; w < F_THREADS / 64; w++) {
      g += s_red[w * RPW + gi];
      u += s_red[w * RPW + ui];
    }
    const uint16_t hb = f32_to_bf16(silu_f32(g) * u);  // h is rounded to bf16, as in the other paths
    s_h[j] = hb;
    hv = bf16_to_f32(hb);
  }
  (void)NKP;
  return hv;
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

// z = RMSNorm(h) -> LDS (bf16) and, for quantised weights, its 32-element
// block sums (the stack-layer counterpart of stage_x).
__device__ __forceinline__ void stage_z(const uint16_t* h, int H, float eps, uint16_t* xs, float* xsum, float* s_n) {
  const int n8 = H >> 3, i = threadIdx.x;
  const uint4 hv = reinterpret_cast<const uint4*>(h)[min(i, n8 - 1)];  // clamped, unconditional
  const float inv = stack_inv(hv, H, eps, s_n);
  if (i < n8) {
    const uint4 v = make_uint4(scale_pair(hv.x, inv), scale_pair(hv.y, inv), scale_pair(hv.z, inv), scale_pair(hv.w, inv));
    reinterpret_cast<uint4*>(xs)[i] = v;
    if (xsum) {
      float s = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
                ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
      s += dpp_f32<DPP_XOR1>(s);
      s += dpp_f32<DPP_XOR2>(s);
      if ((i & 3) == 0) xsum[i >> 2] = s;
    }
  }
}

constexpr int F_NV = 8;  // logits per lane in the top-k: E <= 512 on this path

// Ordered top-k of the token by the whole workgroup (thread t holds expert
// t; E <= F_THREADS), from the tagged logits:
//   1. each thread's 32-bit sortable key (leading bits of the fp64 logit,
//      the low 9 bits replaced by 511 - t: distinct keys that never
//      contradict value order at the bits they keep); the maximum of each
//      16-thread row (the first 32 rows hold the E <= 512 logits);
//   2. tau = the k-th largest row maximum (every wave computes it from LDS:
//      lane r < 32 counts the row maxima above row r's), tv = the smallest
//      fp64 value with tau's leading bits. k rows hold a value >= tv, so
//      every top-k value is >= tv;
//   3. candidates (values >= tv) appended to LDS (one LDS atomic per wave);
//   4. wave 0 ranks the candidates exactly (value, then index): four lanes
//      per candidate when there are at most 16 (the usual case: about 12),
//      one lane per candidate up to 64, else the one-wave top-k over all
//      values (massive ties). The winners land in S.out[0 .. k) in order.
// The gates (block_topk_gates) are not needed to pick the experts, so the
// caller computes them once its weight loads are in flight.
struct BlockTopk {
  double val[F_THREADS];         // every logit (-inf past E), for the tie path
  uint32_t rowmax[F_THREADS / 16];
  uint32_t cnt;                  // candidates appended
  uint32_t pad[3];
  TopkSlot cand[64];
  TopkSlot out[16];
  uint8_t wave_scratch[TOPK_SCRATCH];
};
static_assert(64 * F_NV <= F_THREADS, "one logit per thread");

__device__ __forceinline__ void block_topk(const uint64_t* logits, int E, int k, uint32_t tag, uint32_t* sync,
                                           BlockTopk& S) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // 1. one logit per thread: coherent loads (a line another call left in
  //    this XCD's L2 is never used), clamped and unconditional
  const int e = min(t, E - 1);
  uint64_t wl = ld_word_coherent(logits + 2 * e);
  uint64_t wh = ld_word_coherent(logits + 2 * e + 1);
  if (t == 0) S.cnt = 0;
  settle2(logits + 2 * e, logits + 2 * e + 1, wl, wh, tag, sync);  // the last router rows may be on their way
  const double v = (t < E) ? __longlong_as_double((long long)(((wh & 0xFFFFFFFFull) << 32) | (wl & 0xFFFFFFFFull)))
                           : -__builtin_inf();
  S.val[t] = v;
  const uint32_t key = (sort_key_hi(v) & ~511u) | (uint32_t)(511 - min(t, 511));
  uint32_t m = key;
  m = max(m, (uint32_t)dpp_i32<DPP_XOR1>((int)m));
  m = max(m, (uint32_t)dpp_i32<DPP_XOR2>((int)m));
  m = max(m, (uint32_t)dpp_i32<DPP_HALF_MIRROR>((int)m));
  m = max(m, (uint32_t)dpp_i32<DPP_MIRROR>((int)m));
  if ((lane & 15) == 0) S.rowmax[t >> 4] = m;
  __syncthreads();
  // 2. threshold, 3. candidates (waves holding experts only)
  if (wave * 64 < E) {
    const uint32_t mine = S.rowmax[lane & 31];
    const uint4* rm = reinterpret_cast<const uint4*>(S.rowmax);
    int r0 = 0, r1 = 0;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const uint4 q = rm[j], q2 = rm[j + 1];
      r0 += (int)(q.x > mine) + (int)(q.y > mine) + (int)(q.z > mine) + (int)(q.w > mine);
      r1 += (int)(q2.x > mine) + (int)(q2.y > mine) + (int)(q2.z > mine) + (int)(q2.w > mine);
    }
    const uint64_t sel = __ballot((lane < 32) & (r0 + r1 == k - 1));
    const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)mine, __ffsll((long long)sel) - 1) & ~511u;
    const double tv = key_floor_value(tau);
    // 3. candidates
    const bool cand = (t < E) & (v >= tv);
    const uint64_t bal = __ballot(cand);
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&S.cnt, (uint32_t)__popcll(bal));
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
    const uint32_t pos = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (cand & (pos < 64u)) {
      S.cand[pos].v = v;
      S.cand[pos].i = t;
    }
  }
  __syncthreads();
  // 4. exact order
  if (wave == 0) {
    const int nc = (int)S.cnt;
    if (nc <= 16) {
      const int c = lane >> 2, g = lane & 3;
      const TopkSlot me = S.cand[c < nc ? c : 0];
      int rk = 0;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int j = g + 4 * jj;
        const TopkSlot o = S.cand[j < nc ? j : 0];
        rk += (int)((j < nc) & topk_before(o.v, o.i, me.v, me.i));
      }
      rk += dpp_i32<DPP_XOR1>(rk);
      rk += dpp_i32<DPP_XOR2>(rk);
      if ((g == 0) & (c < nc) & (rk < k)) S.out[rk] = me;
    } else if (nc <= 64) {
      const TopkSlot me = S.cand[lane < nc ? lane : 0];
      int rk = 0;
      for (int j = 0; j < nc; j++) {
        const TopkSlot o = S.cand[j];
        rk += (int)topk_before(o.v, o.i, me.v, me.i);
      }
      if ((lane < nc) & (rk < k)) S.out[rk] = me;
    } else {
      double w[F_NV];
#pragma unroll
      for (int i = 0; i < F_NV; i++) w[i] = S.val[lane + 64 * i];
      wave_topk_order<F_NV>(w, E, k, lane, S.wave_scratch, S.out);
    }
  }
  __syncthreads();
}

// Gates of the k winners by wave 0 into s_idx/s_gate (the workgroup reads
// them after a barrier).
__device__ __forceinline__ void block_topk_gates(const BlockTopk& S, int E, int k, int* s_idx, float* s_gate) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int mi;
    float mg;
    topk_gates(S.out, E, k, lane, mi, mg);
    if (lane < k) {
      s_idx[lane] = mi;
      s_gate[lane] = mg;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K down: one workgroup's columns of a down matrix times its h, for
// all H output rows, as tagged partial words part[row] (fp32 bits). Rows go
// to threads round-robin (lane-consecutive rows read consecutive chunks).
// Columns c0 ..: routed 32 (one quantised chunk per row, or 32 / kchunk
// dense chunks), shared 8 (8 / kchunk chunks). When a row's columns are one
// chunk (quantised routed, bf16 shared) the chunks and scales of the
// thread's rows go to registers while the gate/up rows stream; otherwise the
// rows are loaded once h is ready.
// ---------------------------------------------------------------------------
template <int WT, int NCOL> struct DownPlan {
  static constexpr int KC = kchunk<WT>();
  static constexpr int NCH = NCOL / KC > 0 ? NCOL / KC : 1;  // chunks per row holding the columns
  static constexpr bool PRE = NCH == 1;                      // chunks prefetched into registers
};

// this thread's prefetched rows: chunk and scale per row
template <int WT>
struct DownPre {
  Raw r[F_RPT];
  uint16_t s[F_RPT];  // fp16 bits, converted at the use (a conversion here would wait for the load)
};

// issue the prefetch of this thread's rows (columns from c0) into registers;
// every row slot is filled, with no branch (a load inside a branch makes the
// compiler wait for all loads in flight where the branch joins); rows past H
// load row H - 1 and are not used
template <int WT, int NCOL>
__device__ __forceinline__ void down_prefetch(const uint8_t* __restrict__ d, const uint16_t* __restrict__ ds, int H,
                                              int c0, DownPre<WT>& pre) {
  if constexpr (DownPlan<WT, NCOL>::PRE) {
    const int cb = c0 / DownPlan<WT, NCOL>::KC;  // the chunk column
#pragma unroll
    for (int n = 0; n < F_RPT; n++)
      pre.r[n] = load_chunk<WT>(d, (size_t)cb * H + min((int)threadIdx.x + F_THREADS * n, H - 1));
    if constexpr (is_q<WT>()) {
#pragma unroll
      for (int n = 0; n < F_RPT; n++)
        pre.s[n] = ds[(size_t)cb * H + min((int)threadIdx.x + F_THREADS * n, H - 1)];
    }
  }
}

// partial[row] = scale * (its columns . h), stored as tagged words
template <int WT, int NCOL>
__device__ __forceinline__ void down_store(const uint8_t* __restrict__ d, int H, int c0, const DownPre<WT>& pre,
                                           const uint16_t* s_h, float hsum, float scale, uint64_t* part, uint32_t tag) {
  constexpr int KC = DownPlan<WT, NCOL>::KC;
  constexpr int NCH = DownPlan<WT, NCOL>::NCH;
  if constexpr (DownPlan<WT, NCOL>::PRE && is_q<WT>()) {
    // h (32 bf16) in registers once; every row computed (rows past H hold
    // row H - 1's chunk), only the store is conditional
    const uint4* hp = reinterpret_cast<const uint4*>(s_h);
    const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
    uint32_t magic = BF16_MAGIC2;
    asm volatile("" : "+v"(magic));
#pragma unroll
    for (int n = 0; n < F_RPT; n++) {
      const int row = (int)threadIdx.x + F_THREADS * n;
      const float v = f16_to_f32(pre.s[n]) * qdot32_regs<WT>(pre.r[n], hv, hsum, magic);
      if (row < H) st_word(part + row, __float_as_uint(v * scale), tag);
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < F_RPT; n++) {
    const int row = (int)threadIdx.x + F_THREADS * n;
    if (row < H) {
      float v = 0.0f;
      if constexpr (DownPlan<WT, NCOL>::PRE) {
        if constexpr (is_q<WT>()) v = f16_to_f32(pre.s[n]) * qdot32<WT>(pre.r[n], s_h, hsum);
        else v = ddot<WT>(pre.r[n], s_h, 0.0f);
      } else {
#pragma unroll
        for (int c = 0; c < NCH; c++) v = ddot<WT>(load_chunk<WT>(d, (size_t)(c0 / KC + c) * H + row), s_h + KC * c, v);
      }
      st_word(part + row, __float_as_uint(v * scale), tag);
    }
  }
}

// ---------------------------------------------------------------------------
// Reducer: output rows r0 .. r0 + F_RD - 1, y = sum over the nP partials in
// producer order (shared roles, then routed), each thread summing a fixed
// subset and the workgroup adding the subsets in a fixed order. The reducer
// polls the partial words themselves (no flags): a pass costs one request
// per producer line, as a flag poll would, and the data is there as soon as
// the poll sees it.
// ---------------------------------------------------------------------------
constexpr int F_RD = 16;                   // output rows per reducer
constexpr int F_RG = F_THREADS / F_RD;     // producer groups per reducer (64)

__device__ __forceinline__ void role_reduce(const uint64_t* part, int nP, int H, int r0, uint16_t* __restrict__ y,
                                            float* s_red, uint32_t tag, uint32_t* sync, const StackIo& S) {
  const int rr = threadIdx.x % F_RD, pg = threadIdx.x / F_RD;
  const int row = r0 + rr;
  float acc = 0.0f;
  const int rowc = min(row, H - 1);
  constexpr int NB = 4;  // F_RG * NB >= the producers of the usual shapes: one batch of loads
  for (int p0 = pg; p0 < nP; p0 += F_RG * NB) {
    uint64_t w[NB];
#pragma unroll
    for (int n = 0; n < NB; n++)  // clamped, unconditional loads (see role_router)
      w[n] = ld_word_coherent(part + (size_t)min(p0 + F_RG * n, nP - 1) * H + rowc);
    // words of producers that are not done yet: the wave reloads its whole
    // batch (unconditional loads, one round trip per pass) until every tag
    // is current, so late producers cost one round trip, not one per word
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      bool stale = false;
#pragma unroll
      for (int n = 0; n < NB; n++) stale |= (uint32_t)(w[n] >> 32) != tag;
      if (__builtin_amdgcn_ballot_w64(stale) == 0) break;
      __builtin_amdgcn_s_sleep(2);
      uint64_t r[NB];
#pragma unroll
      for (int n = 0; n < NB; n++) r[n] = ld_word_coherent(part + (size_t)min(p0 + F_RG * n, nP - 1) * H + rowc);
#pragma unroll
      for (int n = 0; n < NB; n++) w[n] = ((uint32_t)(w[n] >> 32) == tag) ? w[n] : r[n];
      if ((++it & 15) == 0 && wall_clock64() - t0 > F_WAIT_TICKS) {
        flag_error(sync, 2u);
        break;
      }
    }
#pragma unroll
    for (int n = 0; n < NB; n++)
      if (p0 + F_RG * n < nP) acc += __uint_as_float((uint32_t)w[n]);
  }
  // a wave holds four producer groups of the same 16 rows (lanes rr + 16j):
  // fold them in the wave ((g0 + g1) + (g2 + g3)), then the wave sums
  static_assert(F_RD == 16, "four groups per wave");
  float a = acc + __shfl_xor(acc, 16, 64);
  a += __shfl_xor(a, 32, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < F_RD) s_red[wave * F_RD + lane] = a;
  __syncthreads();
  if ((int)threadIdx.x < F_RD && row < H) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < F_WAVES; w++) t += s_red[w * F_RD + rr];
    const uint16_t yb = f32_to_bf16(t);
    if (S.h) {
      // stack layer: h = bf16(h + y) for this reducer's rows. Every workgroup
      // that reads h has read it before its output (logits, partials) could
      // reach a reducer, and the reducers wait for all of them.
      S.h[row] = f32_to_bf16(bf16_to_f32(S.h[row]) + bf16_to_f32(yb));
      if (S.y_out) S.y_out[row] = yb;
    } else {
      y[row] = yb;
    }
  }
}

// ---------------------------------------------------------------------------
// LDS: static arrays (x, x block sums, wave partials, top-k scratch) sized
// for H <= F_HMAX.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int WT, int SWT>
__global__ __launch_bounds__(F_THREADS, 4) void k_decode1(LayerDev L, const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ y, int32_t* idx_out, float* gate_out,
                                                       DecodeWs ws, FusedGeo G, StackIo S) {
  __shared__ __align__(16) uint16_t s_x[F_HMAX];
  __shared__ __align__(16) float s_xsum[F_HMAX / 32];
  __shared__ __align__(16) float s_red[F_THREADS];
  __shared__ double s_rt[8];
  __shared__ __align__(16) BlockTopk s_tk;
  __shared__ int s_idx[16];
  __shared__ float s_gate[16];
  __shared__ __align__(16) uint16_t s_h[32];
  __shared__ float s_hsum;
  __shared__ float s_n[4];
  const int H = L.H, I = L.I;
  const bool stk = S.h != nullptr;  // stack layer: the token is h, the activations z = RMSNorm(h)
  const int nP = G.nSG + G.nRG;  // partial producers: shared workgroups, then routed
  // this call's tag: the epoch (stable until every workgroup is done) + 1
  const uint32_t tag = ld_u32(ws.sync + SY_EPOCH + SY_LINE * my_rep()) + 1u;
  uint64_t* tl = reinterpret_cast<uint64_t*>(ws.logits) + (size_t)(tag % F_SLOTS) * SY_NREP * 2 * L.E;
  // flags of the router roles
  uint64_t* fl = ws.flags + (size_t)(tag % F_SLOTS) * G.nR * F_FLAG_STRIDE;
  uint64_t* part = ws.part_words;  // [nP][H]
  int b = blockIdx.x;
  if (b < G.nA) {
    if (b < G.nR) {
      role_router(L, stk ? S.h : x, tl, b, s_rt, tag, stk, S.eps, s_n);
      raise_flag(fl, b, tag);
    }
    if (b < G.nSG) {
      // shared expert, intermediates 16q + 8hf .. +7, right after the router
      // rows (its bytes fill the memory-idle top-k window)
      constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
      const uint16_t* xs = s_x;
      const int q = b >> 1, hf = b & 1;
      if (stk) stage_z(S.h, H, S.eps, s_x, nullptr, s_n);
      else stage_x(x, H, s_x, nullptr);  // after the router's loads (x is then in this XCD's L2)
      __syncthreads();
      DownPre<SW> pre;
      gate_up_h<SW, 16>(L.sgu, nullptr, H, 2 * I, q, hf, xs, nullptr, s_red, s_h,
                        [&] { down_prefetch<SW, 8>(L.sdn, nullptr, H, 16 * q + 8 * hf, pre); });
      __syncthreads();
      down_store<SW, 8>(L.sdn, H, 16 * q + 8 * hf, pre, s_h, 0.0f, 1.0f, part + (size_t)b * H, tag);
    }
  } else if ((b -= G.nA) < G.nRG) {
    // routed slot u, intermediates 32q .. 32q+31
    uint16_t* xs = s_x;
    float* xsum = s_xsum;
    if (stk) stage_z(S.h, H, S.eps, xs, is_q<WT>() ? xsum : nullptr, s_n);
    else stage_x(x, H, xs, is_q<WT>() ? xsum : nullptr);
    wait_flags(fl, G.nR, flags_needed(G.nR), tag, ws.sync);  // (its barrier also publishes xs)
    if (stk && S.z_out && b == 0)
      for (int i = threadIdx.x; i < (H >> 3); i += F_THREADS)
        reinterpret_cast<uint4*>(S.z_out)[i] = reinterpret_cast<const uint4*>(xs)[i];
    block_topk(tl + (size_t)my_rep() * 2 * L.E, L.E, L.k, tag, ws.sync, s_tk);
    const int gpe = I >> 5;
    const int u = b / gpe, q = b - u * gpe;
    const int e = min(max(s_tk.out[u].i, 0), L.E - 1);  // in range whatever the logits held
    const uint8_t* dn = L.dn + (size_t)e * L.dn_stride;
    const uint16_t* dns = is_q<WT>() ? L.dn_s + (size_t)e * L.dn_s_stride : nullptr;
    DownPre<WT> pre;
    if constexpr (!is_q<WT>()) block_topk_gates(s_tk, L.E, L.k, s_idx, s_gate);
    const float hv = gate_up_h<WT, 64>(L.gu + (size_t)e * L.gu_stride,
                                       is_q<WT>() ? L.gu_s + (size_t)e * L.gu_s_stride : nullptr, H, 2 * I, q, 0, xs, xsum,
                                       s_red, s_h, [&] {
                                         down_prefetch<WT, 32>(dn, dns, H, 32 * q, pre);
                                         // the gates, while the weights stream (read after gate_up_h's
                                         // barrier); dense weights have no registers to spare there
                                         if constexpr (is_q<WT>()) block_topk_gates(s_tk, L.E, L.k, s_idx, s_gate);
                                       });
    if (b == 0 && (int)threadIdx.x < L.k) {
      if (idx_out) idx_out[threadIdx.x] = s_idx[threadIdx.x];
      if (gate_out) gate_out[threadIdx.x] = s_gate[threadIdx.x];
    }
    if constexpr (is_q<WT>()) {
      // block sum of the 32 bf16 h values (threads 0..31 of wave 0), fixed order
      float t = hv;
      if (threadIdx.x < 64) {
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
        if (threadIdx.x == 0) s_hsum = t;
      }
    }
    __syncthreads();
    down_store<WT, 32>(dn, H, 32 * q, pre, s_h, is_q<WT>() ? s_hsum : 0.0f, s_gate[u],
                       part + (size_t)(G.nSG + b) * H, tag);
  }
  // reducers: the last nD workgroups of the grid, all routed or extra ones
  const int d = (int)blockIdx.x - ((int)gridDim.x - G.nD);
  if (d >= 0) {
    __syncthreads();  // s_red is reused
    role_reduce(part, nP, H, d * F_RD, y, s_red, tag, ws.sync, S);
  }
  finish(ws.sync);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
size_t decode1_lds(int H, int I, int k, bool has_shared) {
  (void)H; (void)I; (void)k; (void)has_shared;
  return 0;  // static arrays only
}

static int producers(int I, int k, bool has_shared) { return (has_shared ? I / 8 : 0) + k * (I / 32); }

size_t decode1_logit_words(int E) { return (size_t)F_SLOTS * SY_NREP * 2 * E; }

size_t decode1_flag_words(int E, int I, int k, bool has_shared) {
  (void)I; (void)k; (void)has_shared;
  return (size_t)F_SLOTS * ((E + 7) / 8) * F_FLAG_STRIDE;
}

// Workgroups: router/shared, routed, and extra reducers when the reducers
// outnumber the routed workgroups (reducers are the last ones).
static int decode1_grid(int E, int H, int I, int k, bool has_shared) {
  const int nR = (E + 7) / 8, nSG = has_shared ? I / 8 : 0, nRG = k * (I / 32);
  const int nA = nR > nSG ? nR : nSG, nD = (H + F_RD - 1) / F_RD;
  return nA + (nRG > nD ? nRG : nD);
}

// Workgroups that are sure to be resident together: one per CU (the launch
// bounds keep a workgroup within a CU's registers; its LDS is ~24 KB).
// Reducers wait for producers dispatched before and after them, so the
// whole grid must be resident at once.
static int decode1_capacity() {
  static int cap[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cap[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cap[dev] = cus;
  }
  return cap[dev];
}

size_t decode1_part_words(int H, int I, int k, bool has_shared) {
  return (size_t)producers(I, k, has_shared) * H;
}

bool decode1_fits(int E, int H, int I, int k, bool has_shared) {
  // F_NV logits per lane in the top-k, F_RPT down rows per thread (the LDS
  // arrays are sized for H <= F_HMAX), a grid that is resident at once
  return E <= 64 * F_NV && H <= F_HMAX && I <= 1024 && decode1_grid(E, H, I, k, has_shared) <= decode1_capacity();
}

template <int WT, int SWT>
static hipError_t launch_fused_t(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out, float* gate_out,
                                 const DecodeWs& ws, hipStream_t st, const StackIo& S) {
  FusedGeo G;
  G.nR = (L.E + 7) / 8;
  G.nSG = (SWT == MOE_W_NONE) ? 0 : L.I / 8;
  G.nRG = L.k * (L.I / 32);
  G.nA = G.nR > G.nSG ? G.nR : G.nSG;
  G.nD = (L.H + F_RD - 1) / F_RD;
  const size_t lds = decode1_lds(L.H, L.I, L.k, SWT != MOE_W_NONE);
  const int grid = decode1_grid(L.E, L.H, L.I, L.k, SWT != MOE_W_NONE);
  return launch_k(KC_DEC_FUSED, k_decode1<WT, SWT>, dim3(grid), dim3(F_THREADS), lds, st, L, x, y, idx_out, gate_out,
                  ws, G, S);
}

template <int WT>
static hipError_t launch_fused_w(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* io, float* go,
                                 const DecodeWs& ws, hipStream_t st, const StackIo& S) {
  if (L.swt == MOE_W_NONE) return launch_fused_t<WT, MOE_W_NONE>(L, x, y, io, go, ws, st, S);
  if (L.swt == MOE_W_F32) return launch_fused_t<WT, MOE_W_F32>(L, x, y, io, go, ws, st, S);
  return launch_fused_t<WT, MOE_W_BF16>(L, x, y, io, go, ws, st, S);
}

hipError_t launch_decode_fused(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out, float* gate_out,
                               const DecodeWs& ws, hipStream_t st, const StackIo* stack) {
  const StackIo S = stack ? *stack : StackIo{nullptr, nullptr, nullptr, 0.0f};
  switch (L.wt) {
    case MOE_W_Q4: return launch_fused_w<MOE_W_Q4>(L, x, y, idx_out, gate_out, ws, st, S);
    case MOE_W_Q3: return launch_fused_w<MOE_W_Q3>(L, x, y, idx_out, gate_out, ws, st, S);
    case MOE_W_BF16: return launch_fused_w<MOE_W_BF16>(L, x, y, idx_out, gate_out, ws, st, S);
    default: return launch_fused_w<MOE_W_F32>(L, x, y, idx_out, gate_out, ws, st, S);
  }
}

}  // namespace moe
