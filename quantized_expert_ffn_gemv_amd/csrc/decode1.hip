// Batch-1 decode of one MoE layer as a single kernel.
//
// 256 workgroups of 1024 threads, one per CU, all resident at once.
// Workgroups are dealt round-robin over the 8 XCDs, so the workgroups b
// with the same b % 8 ("XCD group") share an XCD and its L2 (the first
// XCD of the deal varies from launch to launch). Back to back, as in a
// graph replay, all XCDs start within ~0.2 us of each other (launched one
// at a time after an idle spell, they start one after another over ~2 us).
// Roles:
//
//   b < nR                 router: rr rows each (rr = 2 for E > 256, else 1;
//                          16 / rr waves a row), fp64 logits (an fp32 weight
//                          times a bf16 activation is exact in fp64), every
//                          workgroup first, so the 4 MiB stream over all CUs.
//   b < nRG                routed: (slot, 32 intermediates) each; ordered
//                          top-k from the logits, fused dequantise-GEMV of
//                          the 64 gate/up rows + SwiGLU -> h (bf16, in LDS),
//                          then the matching 32-column block of the
//                          expert's down matrix (loaded with the gate/up
//                          rows) times h, scaled by the slot's gate: a
//                          partial y over all H rows. Workgroup b < 8 is
//                          also its XCD's forwarder of the logits.
//   sg0 <= b < sg0 + nSG   shared expert, 8 intermediates each: 16 gate/up
//                          rows, SwiGLU -> h, then those 8 columns of the
//                          shared down matrix times h: a partial y over all
//                          H rows (sg0 = nRG rounded up to a multiple of 8);
//                          started once the XCD's logits are forwarded.
//
// The down product is split along the intermediate dimension (split-K), so
// h never leaves the workgroup that made it and the down weights stream in
// the same window as the gate/up weights. The partials are then summed in
// two levels:
//
//   XCD level   every workgroup of XCD group x sums, for H/32 rows, the
//               partials of the producers of its own group, which sit in its
//               XCD's L2 (a group that is split over XCDs would show up as a
//               wait that runs out):
//               producers store them with plain stores and readers load
//               them with L1-missing agent-scope loads, served by that L2,
//               so this hand-off stays inside the XCD (about 0.25 us, no
//               HBM or fabric traffic).
//               The sum goes out as one tagged word per row (agent scope).
//   final       every workgroup sums, for H/256 rows, the 8 XCD sums in XCD
//               order and writes y (a stack layer adds the residual).
//
// Hand-off without cache flushes. Every value passed between workgroups is
// a 64-bit word whose high half is a tag that is new for every call, so a
// reader uses a word only once its tag is current and no release/acquire
// fence (an L2 write-back or invalidate per workgroup) is needed: words that
// cross XCDs are stored and loaded with agent-scope relaxed atomics
// (coherent across the XCDs' L2s word by word), words that stay inside an
// XCD are stored with plain stores into that XCD's L2 and read there. The
// router's logits cross once, to one forwarder per XCD, which copies them
// into its XCD's L2 for the other routed workgroups there.
// Every spin is bounded; one that runs out sets an error bit in the
// workspace (1: logits or the XCD's ready word, 2: the L2 copy of the
// logits, 4: XCD sums' inputs, 8: final sums' inputs) and lets the
// workgroup finish, so the kernel always ends.
//
// The tag is the call count each workgroup keeps for itself: workgroup b
// reads its own counter at the start and writes it back incremented at the
// end. Every call runs every workgroup once, so the 256 counters move in
// lockstep and all workgroups derive the same tag, with no atomic and no
// "last one out" count (256 workgroups finishing together serialised on one
// counter for about 1.6 us). The workspace is ready for the next call (and
// for graph replay) without a memset.
//
// Progress: forwarders wait only for the routers (router rows never wait),
// routed and shared units for their forwarder, XCD sums for producers, final sums for
// XCD sums, so every value gets written once every workgroup is resident;
// the path is taken only when the grid fits the chip at one workgroup per
// CU.
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
constexpr int F_NW = 256;                       // workgroups (one per CU)
constexpr int F_NX = 8;                         // XCDs: workgroup b runs on XCD b % 8
constexpr int F_PX = F_NW / F_NX;               // workgroups per XCD
constexpr int F_RPT = 2;                        // down rows per thread (H <= F_RPT * F_THREADS)
constexpr int F_HMAX = F_RPT * F_THREADS;       // largest H of this path (LDS arrays are sized for it)
constexpr int F_RRMAX = 2;                      // router rows per workgroup (E <= F_NW * F_RRMAX)
constexpr uint64_t F_WAIT_TICKS = 1ull << 25;   // ~0.34 s of the 100 MHz wall clock

// Workspace sync area (uint32 words): the error bits in a line of their own,
// then one call counter per workgroup (8 bytes apart).
constexpr int SY_LINE = 32;                                   // words per line
constexpr int SY_NREP = F_NX;                                 // XCD copies of the logits
constexpr int SY_ERR = 0;
constexpr int SY_COUNT = SY_LINE;                             // + 2 b
constexpr int SY_WORDS = SY_COUNT + 2 * F_NW;                 // 2176 bytes
static_assert(SY_WORDS * 4 <= 4096, "sync area");
constexpr int F_SLOTS = 4;  // logit buffers rotate over this many calls
constexpr int RDY_STRIDE = 16;  // uint64 words between the XCDs' ready words (one 128-byte line each)

struct FusedGeo {
  int rr;    // router rows per workgroup (1 or 2)
  int nR;    // router workgroups: [0, nR), rows rr*b .. rr*b + rr - 1
  int nRG;   // routed units (slot, 32 intermediates): workgroups [0, nRG)
  int sg0;   // shared units (8 intermediates each): workgroups [sg0, sg0 + nSG), sg0 = nRG rounded up to 8
  int nSG;
  int xmask; // XCD groups that hold at least one producer (bit x)
  uint64_t wait_ticks;  // bound of every device-side wait
};
// rank of workgroup b when the workgroups are listed XCD by XCD (the final
// sums give each XCD a contiguous block of rows)
__device__ __forceinline__ int start_rank(int b) { return (b % F_NX) * F_PX + b / F_NX; }
// producer index of workgroup b: shared units first, then routed units; -1 for none
__device__ __forceinline__ int producer_of(int b, const FusedGeo& G) {
  if (b < G.nRG) return G.nSG + b;
  if (b >= G.sg0 && b < G.sg0 + G.nSG) return b - G.sg0;
  return -1;
}

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ld_word_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Words that stay inside one XCD: a plain 8-byte store (through the
// write-through L1 into the XCD's L2, where it stays), read with the
// agent-scope load (sc1: misses the reader's L1 and is served by the L2
// that holds the line). Measured on one XCD: seen ~250 ns after the store,
// against ~450 ns when the store also goes out at agent scope. (An sc0 load
// is not enough: a poll keeps hitting the stale line in the reader's L1.)
__device__ __forceinline__ void st_word_xcd(uint64_t* p, uint32_t payload, uint32_t tag) {
  *p = ((uint64_t)tag << 32) | payload;
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// an fp32 value another workgroup of this XCD stored (misses the L1)
__device__ __forceinline__ float ld_f32_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void flag_error(uint32_t* sync, uint32_t bit) {
  __hip_atomic_fetch_or(sync + SY_ERR, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// A pair of words written together and loaded once: while either tag is
// not current (the producer has not stored them yet), reload both
// (bounded).
__device__ __forceinline__ void settle2(const uint64_t* p0, const uint64_t* p1, uint64_t& w0, uint64_t& w1, uint32_t tag,
                                        uint32_t* sync, uint64_t ticks) {
  if (((uint32_t)(w0 >> 32) != tag) | ((uint32_t)(w1 >> 32) != tag)) {
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(2);
      w0 = ld_word_coherent(p0);
      w1 = ld_word_coherent(p1);
      if (((uint32_t)(w0 >> 32) == tag) & ((uint32_t)(w1 >> 32) == tag)) break;
      if ((++it & 15) == 0 && wall_clock64() - t0 > ticks) {
        flag_error(sync, 2u);
        break;
      }
    }
  }
}

// The logits reach the routed workgroups in two hops. The routers store
// them once, at agent scope (one copy in memory). On each XCD one routed
// workgroup, the forwarder, polls those words (8 KB a round: with 8
// pollers the memory side is not flooded), copies them into its XCD's L2
// with plain stores and then raises the XCD's ready word there (for the
// shared units); the other routed workgroups of the XCD poll the copy's
// last word, inside the XCD, and read the logits from the L2 copy (not
// waiting for the ready word, which follows the forwarder's barrier: 14.16
// -> 14.09 us per token). (When every routed workgroup polled the
// memory copy itself, 8 KB a round each, the polls flooded the memory side
// while the routers were still at work; a counter per XCD group that the
// routers bumped cost an atomic and then a second trip for the logits.)
__device__ __forceinline__ void forward_logits(const uint64_t* mem, uint64_t* xc, uint64_t* rdy, int n, uint32_t tag,
                                               uint32_t* sync, uint64_t ticks) {
  const int t = threadIdx.x, i = min(t, n - 1);
  uint64_t w = ld_word_coherent(mem + i);  // clamped, unconditional
  if (__builtin_amdgcn_ballot_w64(!tag_ok(w, tag)) != 0) {
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(1);
      if (!tag_ok(w, tag)) w = ld_word_coherent(mem + i);
      if (__builtin_amdgcn_ballot_w64(!tag_ok(w, tag)) == 0) break;
      if ((++it & 15) == 0 && wall_clock64() - t0 > ticks) {
        if ((t & 63) == 0) flag_error(sync, 1u);
        break;
      }
    }
  }
  if (t < n) st_word_xcd(xc + t, (uint32_t)w, tag);
  __syncthreads();  // every thread's copy has reached the L2 before the ready word
  if (t == 0) st_word_xcd(rdy, 0u, tag);
}
__device__ __forceinline__ void wait_ready(const uint64_t* rdy, uint32_t tag, uint32_t* sync, uint64_t ticks) {
  if (threadIdx.x < 64) {
    uint64_t w = ld_word_coherent(rdy);
    if (!tag_ok(w, tag)) {
      const uint64_t t0 = wall_clock64();
      int it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(1);
        w = ld_word_coherent(rdy);
        if (tag_ok(w, tag)) break;
        if ((++it & 15) == 0 && wall_clock64() - t0 > ticks) {
          if (threadIdx.x == 0) flag_error(sync, 1u);
          break;
        }
      }
    }
  }
  __syncthreads();
}

// The workgroup's call counter: read at the start (the tag is its value + 1)
// and written back incremented once the workgroup is past all of its waits.
__device__ __forceinline__ uint32_t* my_counter(uint32_t* sync) { return sync + SY_COUNT + 2 * blockIdx.x; }
__device__ __forceinline__ void finish(uint32_t* sync, uint32_t tag) {
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(my_counter(sync), tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// Router: waves w and w + 8 of router workgroup rw compute the two halves of
// the logit of expert 8rw + w (summed in that order). The logits are written
// once per XCD group: the routed workgroups of a group read their own copy,
// so each line has a few readers instead of all of them (lines read by
// hundreds of workgroups at once serve them one after another).
// ---------------------------------------------------------------------------
struct RouterRegs {
  float4 w;
  float bias;
};

// Issue the loads of this workgroup's router rows (with the token's, so that
// both are in flight together): rr rows (1 or 2) of rr*b .. rr*b + rr - 1,
// P = 16 / rr waves per row; wave w takes row w / P and the P-th part
// w % P of its float4 columns, one per lane (H <= F_HMAX: a part holds at
// most 64). Every workgroup issues them, clamped inside the row and masked
// when summed (a load under a branch makes the compiler wait for it where
// the branch joins); a workgroup that is not a router reads the first 16
// bytes of the router.
__device__ __forceinline__ void router_issue(const LayerDev& L, bool act, int rw, int rr, RouterRegs& R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = F_WAVES / rr;
  const int e = rw * rr + wave / P;
  const bool valid = act && e < L.E;
  const int n4 = L.H >> 2;
  const int c = (wave % P) * n4 / P + lane;
  const float4* wr = reinterpret_cast<const float4*>(L.router_w + (size_t)(valid ? e : 0) * L.H);
  R.w = wr[act ? min(c, n4 - 1) : 0];
  // the bias with the weights (a load after the sum would be one more
  // memory round trip on the way to the top-k)
  const float* bp = L.router_b ? L.router_b + (valid ? e : 0) : L.router_w;
  R.bias = *bp;
}

// The logits of the rows from the staged activations xs (LDS, bf16): the P
// parts of a row are summed in part order by the row's first wave; the
// logit goes out as two tagged words (low and high half of the fp64 value)
// in the memory copy.
__device__ __forceinline__ void router_finish(const LayerDev& L, const uint16_t* xs, const RouterRegs& R, int rw, int rr,
                                              uint64_t* logits, double* s_rt, uint32_t tag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = F_WAVES / rr, p = wave % P;
  const int e = rw * rr + wave / P;
  const bool valid = e < L.E;
  const int n4 = L.H >> 2;
  const int c = p * n4 / P + lane;
  const bool in = valid && c < (p + 1) * n4 / P;
  const uint2* xv = reinterpret_cast<const uint2*>(xs);
  // the weights enter the arithmetic only here: without this the compiler
  // converts them to fp64 right where they are loaded, which makes the
  // workgroup wait for them before it stages x
  float4 w = R.w;
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
  float bias = R.bias;
  asm volatile("" : "+v"(bias));
  if (!in) w = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint2 xx = xv[in ? c : 0];
  double a0 = __builtin_fma((double)w.z, (double)bf16_lo(xx.y), (double)w.x * (double)bf16_lo(xx.x));
  double a1 = __builtin_fma((double)w.w, (double)bf16_hi(xx.y), (double)w.y * (double)bf16_hi(xx.x));
  const double part = wave_total_f64(a0 + a1);
  if (lane == 0) s_rt[wave] = part;
  __syncthreads();
  if (p == 0 && valid && lane < 2) {
    double tot = s_rt[wave];
    for (int q = 1; q < P; q++) tot += s_rt[wave + q];
    const uint64_t v = (uint64_t)__double_as_longlong(tot + (L.router_b ? (double)bias : 0.0));
    st_word(logits + 2 * e + lane, lane ? (uint32_t)(v >> 32) : (uint32_t)v, tag);
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

template <int WT, int RPW, typename After, typename Before>
__device__ __forceinline__ float gate_up_h(const uint8_t* __restrict__ gu, const uint16_t* __restrict__ gus, int H, int R,
                                           int q, int hf, const uint16_t* xs, const float* xsum, float* s_red,
                                           uint16_t* s_h, After&& after_first_issue, Before&& before_reduce) {
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
  before_reduce();  // work that needs neither h nor the barrier, done while the waves gather
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
  const int n8 = H >> 3, i = threadIdx.x;  // 16-byte chunks: one per thread (H <= F_HMAX)
  const uint4 v = reinterpret_cast<const uint4*>(x)[min(i, n8 - 1)];  // clamped, unconditional
  if (i < n8) {
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
                                           uint64_t ticks, BlockTopk& S) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // 1. one logit per thread: coherent loads (a line another call left in
  //    this XCD's L2 is never used), clamped; only the waves that hold
  //    experts load (when every thread past E loaded the clamped last word,
  //    the workgroups of an XCD sent ~300 requests for that one line to one
  //    L2 channel, behind which the other words on that channel waited)
  const int e = min(t, E - 1);
  uint64_t wl = 0, wh = 0;
  if (t == 0) S.cnt = 0;
  if (wave * 64 < E) {  // wave-uniform
    wl = ld_word_coherent(logits + 2 * e);
    wh = ld_word_coherent(logits + 2 * e + 1);
    settle2(logits + 2 * e, logits + 2 * e + 1, wl, wh, tag, sync, ticks);  // the last router rows may be on their way
  }
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

// partial[row] = scale * (its columns . h), stored as tagged words that stay
// in this XCD's L2
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
      if (row < H) st_word_xcd(part + row, __float_as_uint(v * scale), tag);
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
      st_word_xcd(part + row, __float_as_uint(v * scale), tag);
    }
  }
}

// A routed unit's Q3 down chunks as bf16 pairs (128 + code), unpacked while
// the workgroup gathers its gate/up sums, so that the VALU work left once h
// is known is the dot products alone (a Q3 pair costs a few operations to
// unpack: 13.58 -> 13.48 us per token; for Q4, one and-or per pair, the
// earlier unpack measured 0.03 us slower and is not used), and their fp16
// scales as fp32.
struct DownPairs {
  uint32_t p[F_RPT][16];
  float s[F_RPT];
};
template <int WT>
__device__ __forceinline__ void down_unpack(const DownPre<WT>& pre, DownPairs& d) {
  static_assert(WT == MOE_W_Q3, "Q3 only");
#pragma unroll
  for (int n = 0; n < F_RPT; n++) {
    q3_pairs<BF16_MAGIC2>(pre.r[n].w[0], pre.r[n].w[1], pre.r[n].w[2], d.p[n]);
    d.s[n] = f16_to_f32(pre.s[n]);
  }
}
// down_store for unpacked chunks: the same sums in the same order as
// qdot32_regs, so the partials are bit for bit those of down_store
template <int WT>
__device__ __forceinline__ void down_store_pairs(const DownPairs& d, int H, const uint16_t* s_h, float hsum, float scale,
                                                 uint64_t* part, uint32_t tag) {
  const uint4* hp = reinterpret_cast<const uint4*>(s_h);
  const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
#pragma unroll
  for (int n = 0; n < F_RPT; n++) {
    const int row = (int)threadIdx.x + F_THREADS * n;
    float c0 = -(128.0f + (float)QOff<WT>::v) * hsum, c1 = 0.0f, c2 = 0.0f, c3 = 0.0f;
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      c0 = dot2_bf16(d.p[n][4 * qq + 0], hv[qq].x, c0);
      c1 = dot2_bf16(d.p[n][4 * qq + 1], hv[qq].y, c1);
      c2 = dot2_bf16(d.p[n][4 * qq + 2], hv[qq].z, c2);
      c3 = dot2_bf16(d.p[n][4 * qq + 3], hv[qq].w, c3);
    }
    const float v = d.s[n] * ((c0 + c1) + (c2 + c3));
    if (row < H) st_word_xcd(part + row, __float_as_uint(v * scale), tag);
  }
}

// ---------------------------------------------------------------------------
// XCD-level sum. Workgroup j of XCD x sums rows r0 .. r0 + H/32 - 1 (r0 =
// j * H/32) over the partials of the producers that run on XCD x (the
// workgroups 8j' + x, j' = 0..31, in j' order), which this XCD's L2 holds.
// Thread t takes row t % 64 and the producers of workgroups j' = t / 64 and
// t / 64 + 16; the 16 groups are added in order. The sums go out as tagged
// words xs[x][row] (agent scope: the final sums read them from every XCD).
// The reader polls the partial words themselves (inside the XCD a poll
// costs L2 requests only).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void role_sum_xcd(const uint64_t* part, uint64_t* xs, const FusedGeo& G, int H, float* s_red,
                                             uint32_t tag, uint32_t* sync) {
  const int x = blockIdx.x % F_NX, j = blockIdx.x / F_NX;
  const int nrow = H / F_PX, r0 = j * nrow;  // H % 32 == 0
  const int rr = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int row = r0 + min(rr, nrow - 1);
  int p[2];
  const uint64_t* pw[2];
  uint64_t w[2];
#pragma unroll
  for (int n = 0; n < 2; n++) {
    p[n] = producer_of(F_NX * (g + 16 * n) + x, G);
    pw[n] = part + (size_t)max(p[n], 0) * H + row;
    w[n] = ld_word_coherent(pw[n]);  // unconditional: a word of a non-producer is not used
  }
  // bounded poll of this thread's stale words (producers still computing)
  bool stale = false;
#pragma unroll
  for (int n = 0; n < 2; n++) stale |= (p[n] >= 0) && !tag_ok(w[n], tag);
  if (__builtin_amdgcn_ballot_w64(stale) != 0) {
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(1);
      // both words again, unconditionally: a load under a branch waits for
      // its answer before the next one is sent
      uint64_t nw[2];
#pragma unroll
      for (int n = 0; n < 2; n++) nw[n] = ld_word_coherent(pw[n]);
      stale = false;
#pragma unroll
      for (int n = 0; n < 2; n++) {
        w[n] = tag_ok(w[n], tag) ? w[n] : nw[n];
        stale |= (p[n] >= 0) && !tag_ok(w[n], tag);
      }
      if (__builtin_amdgcn_ballot_w64(stale) == 0) break;
      if ((++it & 15) == 0 && wall_clock64() - t0 > G.wait_ticks) {
        if ((threadIdx.x & 63) == 0) flag_error(sync, 4u);
        break;
      }
    }
  }
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 2; n++) acc += (p[n] >= 0) ? __uint_as_float((uint32_t)w[n]) : 0.0f;
  s_red[g * 64 + rr] = acc;
  __syncthreads();
  if (rr < nrow && threadIdx.x < 64) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < F_WAVES; q++) t += s_red[q * 64 + rr];
    st_word(xs + (size_t)x * H + r0 + rr, __float_as_uint(t), tag);
  }
}

// ---------------------------------------------------------------------------
// Final sum: rows row0 .. row0 + nr - 1 (nr <= 8) of y = the XCD sums in XCD
// order (XCDs without producers add nothing). Wave 0: lane t takes row t % 8
// and XCD t / 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void role_sum_final(const uint64_t* xs, const FusedGeo& G, int H, int row0, int nr,
                                               uint16_t* __restrict__ y, uint32_t tag, uint32_t* sync,
                                               const StackIo& S) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x, r = lane & 7, q = lane >> 3;
  const bool use = ((G.xmask >> q) & 1) && r < nr;
  const uint64_t* pw = xs + (size_t)q * H + row0 + min(r, max(nr - 1, 0));
  uint64_t w = ld_word_coherent(pw);
  if (__builtin_amdgcn_ballot_w64(use && !tag_ok(w, tag)) != 0) {
    const uint64_t t0 = wall_clock64();
    int it = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(1);
      if (use && !tag_ok(w, tag)) w = ld_word_coherent(pw);
      if (__builtin_amdgcn_ballot_w64(use && !tag_ok(w, tag)) == 0) break;
      if ((++it & 15) == 0 && wall_clock64() - t0 > G.wait_ticks) {
        if (lane == 0) flag_error(sync, 8u);
        break;
      }
    }
  }
  // add the XCDs in order: lanes r + 8q, q = 0..7
  float v = use ? __uint_as_float((uint32_t)w) : 0.0f;
  float t = v;
#pragma unroll
  for (int qq = 1; qq < F_NX; qq++) t += __shfl(v, r + 8 * qq, 64);
  if (lane < nr) {
    const int row = row0 + lane;
    const uint16_t yb = f32_to_bf16(t);
    if (S.h) {
      // stack layer: h = bf16(h + y) for these rows. Every workgroup that
      // reads h has read it before its output (logits, partials) could reach
      // an XCD sum, and the final sums wait for all of those.
      S.h[row] = f32_to_bf16(bf16_to_f32(S.h[row]) + bf16_to_f32(yb));
      if (S.y_out) S.y_out[row] = yb;
    } else {
      y[row] = yb;
    }
  }
}

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
  __shared__ double s_rt[F_WAVES];
  __shared__ __align__(16) BlockTopk s_tk;
  __shared__ int s_idx[16];
  __shared__ float s_gate[16];
  __shared__ __align__(16) uint16_t s_h[32];
  __shared__ float s_hsum;
  __shared__ float s_n[4];
  const int H = L.H, I = L.I;
  const bool stk = S.h != nullptr;  // stack layer: the token is h, the activations z = RMSNorm(h)
  const int b = blockIdx.x, rank = start_rank(b);
  // this call's tag: the workgroup's own call count + 1 (the same in every workgroup)
  const uint32_t tag = ld_u32(my_counter(ws.sync)) + 1u;
  // this call's logits: the memory copy, then one copy per XCD
  uint64_t* tl = reinterpret_cast<uint64_t*>(ws.logits) + (size_t)(tag % F_SLOTS) * (1 + SY_NREP) * 2 * L.E;
  uint64_t* tx = tl + (size_t)(1 + b % F_NX) * 2 * L.E;
  uint64_t* rdy = reinterpret_cast<uint64_t*>(ws.ctr) + (size_t)(b % F_NX) * RDY_STRIDE;
  uint64_t* part = ws.part_words;  // [nSG + nRG][H], in the producers' XCD L2s
  const bool is_router = b < G.nR;
  const bool is_routed = b < G.nRG;
  const bool is_shared = b >= G.sg0 && b < G.sg0 + G.nSG;
  // the token and the router rows are loaded together (straight-line code:
  // see router_issue), then x (or z = RMSNorm(h)) goes to LDS. A workgroup
  // without a role in a stack layer reads no part of h (its source is the
  // router's first bytes): every reader of h must precede the writers of h.
  const bool has_role = is_router || is_routed || is_shared;
  const uint16_t* src = (has_role || !stk) ? (stk ? S.h : x) : reinterpret_cast<const uint16_t*>(L.router_w);
  const int n8 = H >> 3;
  const uint4 tv = reinterpret_cast<const uint4*>(src)[min((int)threadIdx.x, n8 - 1)];  // clamped, unconditional
  RouterRegs rrg;
  router_issue(L, is_router, b, G.rr, rrg);
  {
    uint4 v = tv;
    if (stk) {
      const float inv = stack_inv(tv, H, S.eps, s_n);
      v = make_uint4(scale_pair(tv.x, inv), scale_pair(tv.y, inv), scale_pair(tv.z, inv), scale_pair(tv.w, inv));
    }
    if ((int)threadIdx.x < n8) {
      reinterpret_cast<uint4*>(s_x)[threadIdx.x] = v;
      if (is_routed && is_q<WT>()) {
        // 32-element block sums: chunks 4b..4b+3 are lanes 4b'..4b'+3 of one quad
        float sm = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
                   ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
        sm += dpp_f32<DPP_XOR1>(sm);
        sm += dpp_f32<DPP_XOR2>(sm);
        if ((threadIdx.x & 3) == 0) s_xsum[threadIdx.x >> 2] = sm;
      }
    }
  }
  __syncthreads();
  if (is_router) router_finish(L, s_x, rrg, b, G.rr, tl, s_rt, tag);
  if (is_shared) {
    // shared expert, intermediates 8su .. 8su+7 (needed only by the sums).
    // Its 6 MB stream starts once the XCD's logits are forwarded: loads in
    // flight slow the routers' logit words on their way across the XCDs,
    // which are on the critical path (14.34 -> 14.22 us per token; with the
    // routed experts' rows loaded ahead of the routing instead, a probe with
    // the experts known in advance, 14.36 -> 15.05 us). Only when every XCD
    // has a forwarder.
    if (G.nRG >= F_NX) wait_ready(rdy, tag, ws.sync, G.wait_ticks);
    constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
    const int su = b - G.sg0;
    const int q = su >> 1, hf = su & 1;
    DownPre<SW> pre;
    gate_up_h<SW, 16>(L.sgu, nullptr, H, 2 * I, q, hf, s_x, nullptr, s_red, s_h,
                      [&] { down_prefetch<SW, 8>(L.sdn, nullptr, H, 16 * q + 8 * hf, pre); }, [] {});
    __syncthreads();
    down_store<SW, 8>(L.sdn, H, 16 * q + 8 * hf, pre, s_h, 0.0f, 1.0f, part + (size_t)su * H, tag);
  }
  const int ru = b;  // routed unit of this workgroup (if < nRG)
  if (is_routed) {
    // routed slot u, intermediates 32q .. 32q+31
    uint16_t* xs = s_x;
    float* xsum = s_xsum;
    if (stk && S.z_out && ru == 0)
      for (int i = threadIdx.x; i < (H >> 3); i += F_THREADS)
        reinterpret_cast<uint4*>(S.z_out)[i] = reinterpret_cast<const uint4*>(xs)[i];
    // this XCD's forwarder copies the logits; the other routed workgroups
    // wait for the copy's last word itself rather than for the ready word
    // (which the forwarder raises only once all of its copy stores have
    // completed): block_topk then polls any word of the copy that is still
    // on its way
    if (ru < F_NX) forward_logits(tl, tx, rdy, 2 * L.E, tag, ws.sync, G.wait_ticks);
    else wait_ready(tx + 2 * L.E - 1, tag, ws.sync, G.wait_ticks);
    block_topk(tx, L.E, L.k, tag, ws.sync, G.wait_ticks, s_tk);
    const int gpe = I >> 5;
    const int u = ru / gpe, q = ru - u * gpe;
    const int e = min(max(s_tk.out[u].i, 0), L.E - 1);  // in range whatever the logits held
    const uint8_t* dn = L.dn + (size_t)e * L.dn_stride;
    const uint16_t* dns = is_q<WT>() ? L.dn_s + (size_t)e * L.dn_s_stride : nullptr;
    DownPre<WT> pre;
    DownPairs dp;  // Q3: the down chunks as bf16 pairs, unpacked before h is known
    if constexpr (!is_q<WT>()) block_topk_gates(s_tk, L.E, L.k, s_idx, s_gate);
    const float hv = gate_up_h<WT, 64>(
        L.gu + (size_t)e * L.gu_stride, is_q<WT>() ? L.gu_s + (size_t)e * L.gu_s_stride : nullptr, H, 2 * I, q, 0, xs,
        xsum, s_red, s_h,
        [&] {
          down_prefetch<WT, 32>(dn, dns, H, 32 * q, pre);
          // the gates, while the weights stream (read after gate_up_h's
          // barrier); dense weights have no registers to spare there
          if constexpr (is_q<WT>()) block_topk_gates(s_tk, L.E, L.k, s_idx, s_gate);
        },
        [&] {
          if constexpr (WT == MOE_W_Q3) down_unpack<WT>(pre, dp);
        });
    if (ru == 0 && (int)threadIdx.x < L.k) {
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
    if constexpr (WT == MOE_W_Q3)
      down_store_pairs<WT>(dp, H, s_h, s_hsum, s_gate[u], part + (size_t)(G.nSG + ru) * H, tag);
    else
      down_store<WT, 32>(dn, H, 32 * q, pre, s_h, is_q<WT>() ? s_hsum : 0.0f, s_gate[u],
                         part + (size_t)(G.nSG + ru) * H, tag);
  }
  // XCD sums (XCDs that hold producers), then the final rows
  if ((G.xmask >> (b % F_NX)) & 1) {
    __syncthreads();  // s_red is reused
    role_sum_xcd(part, ws.xsum_words, G, H, s_red, tag, ws.sync);
  }
  const int row0 = rank * H / F_NW, nr = (rank + 1) * H / F_NW - row0;
  if (nr > 0) role_sum_final(ws.xsum_words, G, H, row0, nr, y, tag, ws.sync, S);
  finish(ws.sync, tag);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static uint64_t g_wait_ticks = F_WAIT_TICKS;
void decode1_set_wait_ticks(uint64_t ticks) { g_wait_ticks = ticks ? ticks : F_WAIT_TICKS; }

size_t decode1_lds(int H, int I, int k, bool has_shared) {
  (void)H; (void)I; (void)k; (void)has_shared;
  return 0;  // static arrays only
}

static int producers(int I, int k, bool has_shared) { return (has_shared ? I / 8 : 0) + k * (I / 32); }

size_t decode1_logit_words(int E) { return (size_t)F_SLOTS * (1 + SY_NREP) * 2 * E; }

size_t decode1_part_words(int H, int I, int k, bool has_shared) { return (size_t)producers(I, k, has_shared) * H; }

size_t decode1_xsum_words(int H) { return (size_t)F_NX * H; }

size_t decode1_counter_words() { return (size_t)F_NX * RDY_STRIDE * 2; }  // the XCDs' ready words

// Workgroups that are sure to be resident together: one per CU (the launch
// bounds keep a workgroup within a CU's registers; its LDS is ~24 KB).
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

// The kernel's workgroups wait for each other, so all of them must be
// resident at once: a build that spills to scratch memory is not used (the
// scratch a wave needs is handed out as waves launch and can hold some of
// them back until others have finished).
template <typename K>
static bool no_scratch(K kernel) {
  hipFuncAttributes a;
  return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(kernel)) == hipSuccess && a.localSizeBytes == 0;
}
static bool decode1_no_scratch() {
  static const bool ok = no_scratch(k_decode1<MOE_W_Q4, MOE_W_NONE>) && no_scratch(k_decode1<MOE_W_Q4, MOE_W_F32>) &&
                         no_scratch(k_decode1<MOE_W_Q4, MOE_W_BF16>) && no_scratch(k_decode1<MOE_W_Q3, MOE_W_NONE>) &&
                         no_scratch(k_decode1<MOE_W_Q3, MOE_W_F32>) && no_scratch(k_decode1<MOE_W_Q3, MOE_W_BF16>) &&
                         no_scratch(k_decode1<MOE_W_BF16, MOE_W_NONE>) && no_scratch(k_decode1<MOE_W_BF16, MOE_W_F32>) &&
                         no_scratch(k_decode1<MOE_W_BF16, MOE_W_BF16>) && no_scratch(k_decode1<MOE_W_F32, MOE_W_NONE>) &&
                         no_scratch(k_decode1<MOE_W_F32, MOE_W_F32>) && no_scratch(k_decode1<MOE_W_F32, MOE_W_BF16>);
  return ok;
}

bool decode1_fits(int E, int H, int I, int k, bool has_shared) {
  // F_NV logits per lane in the top-k, F_RPT down rows per thread (the LDS
  // arrays are sized for H <= F_HMAX), at most one shared or routed unit per
  // workgroup, and a grid that is resident at once
  const int nSG = has_shared ? I / 8 : 0, nRG = k * (I / 32);
  const int sg0 = (nRG + F_NX - 1) / F_NX * F_NX;
  return E <= 64 * F_NV && E <= F_NW * F_RRMAX && H <= F_HMAX && I <= 1024 && sg0 + nSG <= F_NW &&
         F_NW <= decode1_capacity() && decode1_no_scratch();
}

template <int WT, int SWT>
static hipError_t launch_fused_t(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out, float* gate_out,
                                 const DecodeWs& ws, hipStream_t st, const StackIo& S) {
  FusedGeo G;
  G.rr = L.E > F_NW ? 2 : 1;
  G.nR = (L.E + G.rr - 1) / G.rr;
  G.nSG = (SWT == MOE_W_NONE) ? 0 : L.I / 8;
  G.nRG = L.k * (L.I / 32);
  G.sg0 = (G.nRG + F_NX - 1) / F_NX * F_NX;
  G.xmask = 0;
  for (int b = 0; b < F_NW; b++)
    if (b < G.nRG || (b >= G.sg0 && b < G.sg0 + G.nSG)) G.xmask |= 1 << (b % F_NX);
  G.wait_ticks = g_wait_ticks;
  return launch_k(KC_DEC_FUSED, k_decode1<WT, SWT>, dim3(F_NW), dim3(F_THREADS), 0, st, L, x, y, idx_out, gate_out,
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


// ===========================================================================
// Batched decode, B = 2..8 tokens, as a single kernel
// ===========================================================================
// The batch-1 kernel's structure with the batch folded in:
//   - router rows (every workgroup, as at batch 1) dotted with all B tokens;
//   - each XCD's forwarder (b < 8) computes the B ordered top-k's (one wave
//     per token), the batch's unique experts in order of first appearance
//     (slot order t k + r) with the mask of the tokens that chose each, and
//     hands that on inside its XCD as tagged words (FB_NRES of them);
//   - shared units (8 intermediates each) on workgroups 8 .. 8 + nSG - 1,
//     for all B tokens, while the routing is being made;
//   - routed units (unique expert j, 32 intermediates q), nu * I/32 of
//     them, dealt round-robin from workgroup 8 + nSG on: an expert chosen by
//     several tokens is streamed once and dotted with each of them;
//   - every workgroup adds its units' down products into a partial y per
//     token (2 rows per thread and token, registers), written once for the
//     tokens it touched as plain fp32 (no tags: 4 bytes a value), then the
//     workgroup's done word; the XCD-level and final sums are those of batch
//     1, per token.
// Waits: forwarders for the routers, the others for their forwarder's
// routing words, XCD sums for the done words of their XCD's producers
// (then their partials), final sums for the XCD sums.
constexpr int FB_MAXB = 8;
constexpr int FB_XMAX = 16384;                         // B H: bf16 values of the staged batch
constexpr int FB_SLOTS = FB_MAXB * 16;                 // B k <= 128
constexpr int FB_RES_U = 1;                            // word 1 + j: expert | token mask << 16
constexpr int FB_RES_I = FB_RES_U + FB_SLOTS;          // word FB_RES_I + s: expert of slot s = t k + r | its unique index << 16
constexpr int FB_RES_G = FB_RES_I + FB_SLOTS;          // word FB_RES_G + s: its gate (fp32 bits)
constexpr int FB_NRES = FB_RES_G + FB_SLOTS;           // 385 words (word 0: nu)
constexpr int FB_RES_STRIDE = 512;                     // words per XCD
static_assert(FB_NRES <= FB_RES_STRIDE && FB_NRES <= F_THREADS, "routing words");
constexpr int FB_RED = FB_MAXB * F_WAVES * 64;         // floats of the reduction area (also the top-k scratch)
static_assert(FB_MAXB * TOPK_SCRATCH <= FB_RED * 4, "top-k scratch fits the reduction area");

struct BatchGeo {
  int B;
  int rr, nR;   // router rows per workgroup, router workgroups
  int nSG;      // shared units: workgroups 8 .. 8 + nSG - 1
  int gpe;      // routed units per expert (I / 32)
  int uoff;     // routed unit u runs on workgroup (uoff + u) % 256
  uint64_t wait_ticks;
};

// Router rows dotted with all B tokens: the parts of a row are summed in
// part order by the row's first wave, per token (lanes 2t, 2t + 1 store
// token t's low and high words).
template <int MAXB>
__device__ __forceinline__ void router_finish_b(const LayerDev& L, const uint16_t* xs, int B, const RouterRegs& R,
                                                int rw, int rr, uint64_t* logits, double* s_rt, uint32_t tag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = F_WAVES / rr, p = wave % P;
  const int e = rw * rr + wave / P;
  const bool valid = e < L.E;
  const int n4 = L.H >> 2;
  const int c = p * n4 / P + lane;
  const bool in = valid && c < (p + 1) * n4 / P;
  float4 w = R.w;
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
  float bias = R.bias;
  asm volatile("" : "+v"(bias));
  if (!in) w = make_float4(0.f, 0.f, 0.f, 0.f);
  // all MAXB tokens at once (tokens past B repeat the last one and are not
  // stored), so that their dependent DPP sums interleave instead of running
  // one token after another; each 16-lane row sum goes to LDS and the
  // row-0 wave of the row adds them as ((r0 + r1) + (r2 + r3)), part by
  // part: the association of the batch-1 router
  double v[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    const int tt = min(t, B - 1);
    const uint2 xx = reinterpret_cast<const uint2*>(xs + (size_t)tt * L.H)[in ? c : 0];
    const double a0 = __builtin_fma((double)w.z, (double)bf16_lo(xx.y), (double)w.x * (double)bf16_lo(xx.x));
    const double a1 = __builtin_fma((double)w.w, (double)bf16_hi(xx.y), (double)w.y * (double)bf16_hi(xx.x));
    v[t] = a0 + a1;
  }
#pragma unroll
  for (int t = 0; t < MAXB; t++) v[t] = sum16_f64(v[t]);
  if ((lane & 15) == 0) {
#pragma unroll
    for (int t = 0; t < MAXB; t++)
      if (t < B) s_rt[((size_t)wave * MAXB + t) * 4 + (lane >> 4)] = v[t];
  }
  __syncthreads();
  if (p == 0 && valid && lane < 2 * B) {
    const int t = lane >> 1;
    double tot = 0.0;
    for (int q = 0; q < P; q++) {
      const double* r4 = s_rt + ((size_t)(wave + q) * MAXB + t) * 4;
      const double part = (r4[0] + r4[1]) + (r4[2] + r4[3]);
      tot = q ? tot + part : part;
    }
    const uint64_t bits = (uint64_t)__double_as_longlong(tot + (L.router_b ? (double)bias : 0.0));
    st_word(logits + (size_t)t * 2 * L.E + 2 * e + (lane & 1), (lane & 1) ? (uint32_t)(bits >> 32) : (uint32_t)bits, tag);
  }
}

// Forwarder: the ordered top-k of token t by wave t (the memory copy of its
// logits, polled until every word is current; bounded), then the batch's
// unique experts and masks, published into this XCD's L2 (every word, every
// call, so the readers can check every tag).
template <int MAXB>
__device__ __forceinline__ void fwd_routing_b(const LayerDev& L, const uint64_t* logits, int B, uint32_t tag,
                                              uint32_t* sync, uint64_t ticks, uint8_t* scratch, int* s_mark,
                                              int* s_nu, int* s_uexp, uint32_t* s_umask,
                                              int* s_sidx, int* s_suid, float* s_sgate, uint64_t* res,
                                              int32_t* idx_out, float* gate_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t0 = threadIdx.x;
  const int E = L.E, k = L.k, nslot = B * k;
  if (wave >= B) {
    // the waves without a token clear the union's arrays meanwhile
    const int ct = t0 - 64 * B, nct = F_THREADS - 64 * B;
    for (int e = ct; e < E; e += nct) s_mark[e] = 0x7FFFFFFF;
    if (ct < FB_SLOTS) s_umask[ct] = 0u;
  }
  if constexpr (MAXB == 8) {
    // B >= 6: wave 0 first waits for token 0's words alone (8 KB a round,
    // where every wave polling its own token sends B times that): each
    // router row stores the words of all B tokens in one instruction, so
    // once token 0's are current the others are too, and each wave's own
    // load below normally finds its words current (else it polls them).
    // Zipf B = 8: 49.0 -> 47.6 us per call. At B <= 5 the barrier costs more
    // than the smaller rounds save.
    if (B >= 6) {
      if (wave == 0) {
        uint64_t w[F_NV];
#pragma unroll
        for (int i = 0; i < F_NV; i++) w[i] = ld_word_coherent(logits + 2 * min(lane + 64 * i, E - 1) + 1);
        bool stale = false;
#pragma unroll
        for (int i = 0; i < F_NV; i++) stale |= !tag_ok(w[i], tag);
        if (__builtin_amdgcn_ballot_w64(stale) != 0) {
          const uint64_t c0 = wall_clock64();
          int it = 0;
          while (true) {
            __builtin_amdgcn_s_sleep(2);
            uint64_t n[F_NV];
#pragma unroll
            for (int i = 0; i < F_NV; i++) n[i] = ld_word_coherent(logits + 2 * min(lane + 64 * i, E - 1) + 1);
            stale = false;
#pragma unroll
            for (int i = 0; i < F_NV; i++) {
              w[i] = tag_ok(w[i], tag) ? w[i] : n[i];
              stale |= !tag_ok(w[i], tag);
            }
            if (__builtin_amdgcn_ballot_w64(stale) == 0) break;
            if ((++it & 15) == 0 && wall_clock64() - c0 > ticks) {
              if (lane == 0) flag_error(sync, 2u);
              break;
            }
          }
        }
      }
      __syncthreads();
    }
  }
  if (wave < B) {
    const uint64_t* lg = logits + (size_t)wave * 2 * E;
    uint64_t wl[F_NV], wh[F_NV];
#pragma unroll
    for (int i = 0; i < F_NV; i++) {
      const int e = min(lane + 64 * i, E - 1);
      wl[i] = ld_word_coherent(lg + 2 * e);
      wh[i] = ld_word_coherent(lg + 2 * e + 1);
    }
    bool stale = false;
#pragma unroll
    for (int i = 0; i < F_NV; i++) stale |= !tag_ok(wl[i], tag) || !tag_ok(wh[i], tag);
    if (__builtin_amdgcn_ballot_w64(stale) != 0) {
      const uint64_t c0 = wall_clock64();
      int it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(2);
        uint64_t nl[F_NV], nh[F_NV];
#pragma unroll
        for (int i = 0; i < F_NV; i++) {
          const int e = min(lane + 64 * i, E - 1);
          nl[i] = ld_word_coherent(lg + 2 * e);
          nh[i] = ld_word_coherent(lg + 2 * e + 1);
        }
        stale = false;
#pragma unroll
        for (int i = 0; i < F_NV; i++) {
          wl[i] = tag_ok(wl[i], tag) ? wl[i] : nl[i];
          wh[i] = tag_ok(wh[i], tag) ? wh[i] : nh[i];
          stale |= !tag_ok(wl[i], tag) || !tag_ok(wh[i], tag);
        }
        if (__builtin_amdgcn_ballot_w64(stale) == 0) break;
        if ((++it & 15) == 0 && wall_clock64() - c0 > ticks) {
          if (lane == 0) flag_error(sync, 2u);
          break;
        }
      }
    }
    double v[F_NV];
#pragma unroll
    for (int i = 0; i < F_NV; i++)
      v[i] = (lane + 64 * i < E) ? __longlong_as_double((long long)(((wh[i] & 0xFFFFFFFFull) << 32) | (wl[i] & 0xFFFFFFFFull)))
                                 : -__builtin_inf();
    int mi;
    float mg;
    wave_topk<F_NV>(v, E, k, lane, scratch + (size_t)wave * TOPK_SCRATCH, mi, mg);
    if (lane < k) {
      s_sidx[wave * k + lane] = mi;
      s_sgate[wave * k + lane] = mg;
    }
  }
  // unique experts in slot order of first appearance, and their token masks:
  // the first slot of each expert (LDS atomicMin), then every wave forms the
  // first-appearance masks of all B k <= 128 slots itself (two ballots), so
  // each slot finds its expert's unique index with two popcounts and no
  // further exchange (three barriers in all)
  __syncthreads();
  if (t0 < nslot) atomicMin(&s_mark[s_sidx[t0]], t0);
  __syncthreads();
  const int j0 = min(lane, nslot - 1), j1 = min(64 + lane, nslot - 1);
  const uint64_t m0 = __builtin_amdgcn_ballot_w64((lane < nslot) & (s_mark[s_sidx[j0]] == lane));
  const uint64_t m1 = __builtin_amdgcn_ballot_w64((64 + lane < nslot) & (s_mark[s_sidx[j1]] == 64 + lane));
  const int n0 = __popcll(m0), nu = n0 + __popcll(m1);
  if (t0 < nslot) {
    const int f = s_mark[s_sidx[t0]];  // first slot of this slot's expert (<= t0)
    const int u = f < 64 ? __popcll(m0 & ((1ull << f) - 1ull)) : n0 + __popcll(m1 & ((1ull << (f - 64)) - 1ull));
    if (f == t0) s_uexp[u] = s_sidx[t0];
    atomicOr(&s_umask[u], 1u << (t0 / k));
    s_suid[t0] = u;
  }
  if (t0 == 0) *s_nu = nu;
  __syncthreads();
  if (t0 < FB_NRES) {
    uint32_t pl = 0u;
    if (t0 == 0) {
      pl = (uint32_t)nu;
    } else if (t0 < FB_RES_I) {
      const int j = t0 - FB_RES_U;
      pl = j < nu ? ((uint32_t)s_uexp[j] | (s_umask[j] << 16)) : 0u;
    } else if (t0 < FB_RES_G) {
      const int sl = t0 - FB_RES_I;
      pl = sl < nslot ? ((uint32_t)s_sidx[sl] | ((uint32_t)s_suid[sl] << 16)) : 0u;
    } else {
      const int sl = t0 - FB_RES_G;
      pl = sl < nslot ? __float_as_uint(s_sgate[sl]) : 0u;
    }
    st_word_xcd(res + t0, pl, tag);
  }
  if (idx_out && t0 < nslot) idx_out[t0] = s_sidx[t0];
  if (gate_out && t0 < nslot) gate_out[t0] = s_sgate[t0];
}

// The other workgroups: the XCD's routing words (bounded poll), into LDS.
__device__ __forceinline__ void wait_routing_b(const LayerDev& L, const uint64_t* res, int B, uint32_t tag,
                                               uint32_t* sync, uint64_t ticks, int* s_nu, int* s_uexp,
                                               uint32_t* s_umask, int* s_sidx, int* s_suid, float* s_sgate) {
  const int t0 = threadIdx.x;
  if (t0 < FB_NRES) {
    uint64_t w = ld_word_coherent(res + t0);
    if (__builtin_amdgcn_ballot_w64(!tag_ok(w, tag)) != 0) {
      const uint64_t c0 = wall_clock64();
      int it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(1);
        const uint64_t nw = ld_word_coherent(res + t0);
        w = tag_ok(w, tag) ? w : nw;
        if (__builtin_amdgcn_ballot_w64(!tag_ok(w, tag)) == 0) break;
        if ((++it & 15) == 0 && wall_clock64() - c0 > ticks) {
          if ((t0 & 63) == 0) flag_error(sync, 1u);
          break;
        }
      }
    }
    const uint32_t pl = (uint32_t)w;
    // clamped: in range whatever the words held
    if (t0 == 0) {
      *s_nu = (int)min(pl, (uint32_t)(B * L.k));
    } else if (t0 < FB_RES_I) {
      s_uexp[t0 - FB_RES_U] = min((int)(pl & 0xFFFFu), L.E - 1);
      s_umask[t0 - FB_RES_U] = pl >> 16;
    } else if (t0 < FB_RES_G) {
      s_sidx[t0 - FB_RES_I] = (int)min(pl & 0xFFFFu, (uint32_t)(L.E - 1));
      s_suid[t0 - FB_RES_I] = (int)min(pl >> 16, (uint32_t)(FB_SLOTS - 1));
    } else {
      s_sgate[t0 - FB_RES_G] = __uint_as_float(pl);
    }
  }
  __syncthreads();
}

template <int WT>
__device__ __forceinline__ void qunpack32_m(const Raw& r, uint32_t (&p)[16], uint32_t magic) {
  if constexpr (WT == MOE_W_Q4) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int t = 0; t < 4; t++) p[4 * j + t] = ((r.w[j] >> (4 * t)) & 0x000F000Fu) | magic;
  } else {
    (void)magic;
    q3_pairs<BF16_MAGIC2>(r.w[0], r.w[1], r.w[2], p);
  }
}

// gate_up_h for the tokens in `mask` (of B): each chunk is unpacked once and
// dotted with each of them; token t's h goes to s_hb[32 t + j], j < RPW / 2.
// s_red holds [token][wave][RPW] row sums.
template <int WT, int RPW, int MAXB, typename After>
__device__ __forceinline__ void gate_up_hb(const uint8_t* __restrict__ gu, const uint16_t* __restrict__ gus, int H, int R,
                                           int q, int hf, const uint16_t* xs, const float* xsum, int B, uint32_t mask,
                                           float* s_red, uint16_t* s_hb, After&& after_first_issue) {
  constexpr int KC = kchunk<WT>();
  constexpr int NKP = F_THREADS / RPW;
  constexpr int NB = F_GU_NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane % RPW;
  const int kp = lane / RPW + (64 / RPW) * wave;
  const int row = (RPW == 64) ? 64 * q + rr : 32 * q + 8 * hf + (rr & 7) + ((rr >> 3) << 4);
  const int nc = H / KC, nb = H >> 5;
  uint32_t magic = BF16_MAGIC2;
  asm volatile("" : "+v"(magic));
  constexpr int NBATCH = (F_HMAX / KC + NKP * NB - 1) / (NKP * NB);
  float acc[MAXB];
#pragma unroll
  for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
#pragma unroll
  for (int bt = 0; bt < NBATCH; bt++) {
    const int c0 = bt * NKP * NB;
    Raw raw[NB];
    uint16_t sc[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const size_t o = (size_t)min(c0 + kp + NKP * i, nc - 1) * R + row;
      raw[i] = load_chunk<WT>(gu, o);
      if constexpr (is_q<WT>()) sc[i] = gus[o];
    }
    if (bt == 0) after_first_issue();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const bool in = c0 + kp + NKP * i < nc;
      const int c = min(c0 + kp + NKP * i, nc - 1);
      if constexpr (is_q<WT>()) {
        uint32_t pr[16];
        qunpack32_m<WT>(raw[i], pr, magic);
        const float s = in ? f16_to_f32(sc[i]) : 0.0f;
#pragma unroll
        for (int t = 0; t < MAXB; t++)
          if (t < B && ((mask >> t) & 1u))
            acc[t] = __builtin_fmaf(s, qdot32_p<WT>(pr, xs + (size_t)t * H + 32 * c, xsum[t * nb + c]), acc[t]);
      } else {
#pragma unroll
        for (int t = 0; t < MAXB; t++)
          if (t < B && ((mask >> t) & 1u)) {
            const float d = ddot<WT>(raw[i], xs + (size_t)t * H + (size_t)c * KC, 0.0f);
            acc[t] += in ? d : 0.0f;
          }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXB; t++) {
    if (t < B && ((mask >> t) & 1u)) {
      float a = acc[t];
      if constexpr (RPW == 16) a += __shfl_xor(a, 16, 64);
      if constexpr (RPW <= 32) a += __shfl_xor(a, 32, 64);
      if (lane < RPW) s_red[(t * F_WAVES + wave) * RPW + rr] = a;
    }
  }
  __syncthreads();
  {
    const int i = threadIdx.x, hpt = RPW / 2;
    const int t = i / hpt, j = i - t * hpt;
    if (t < B && ((mask >> t) & 1u)) {
      const int gi = (RPW == 16) ? j : 32 * (j >> 4) + (j & 15);
      const int ui = (RPW == 16) ? j + 8 : gi + 16;
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int w = 0; w < F_WAVES; w++) {
        g += s_red[(t * F_WAVES + w) * RPW + gi];
        u += s_red[(t * F_WAVES + w) * RPW + ui];
      }
      s_hb[32 * t + j] = f32_to_bf16(silu_f32(g) * u);
    }
  }
  __syncthreads();
}

// A routed unit's gate/up, split so that the next unit's loads can be issued
// while this one is still being computed: 64 rows (lane l of wave w: row
// 64q + l, chunks w + 16 i), one batch of F_GU_NB chunks per thread
// (H <= F_HMAX = 16 x F_GU_NB x 32).
static_assert(F_HMAX / 32 == 16 * F_GU_NB, "one batch of gate/up loads per routed unit");
template <int WT>
struct GuRegs {
  Raw raw[F_GU_NB];
  uint16_t sc[F_GU_NB];  // fp16 bits
};
template <int WT>
__device__ __forceinline__ void gu_issue64(const uint8_t* __restrict__ gu, const uint16_t* __restrict__ gus, int H,
                                           int R, int q, GuRegs<WT>& g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = 64 * q + lane, nc = H >> 5;
#pragma unroll
  for (int i = 0; i < F_GU_NB; i++) {
    const size_t o = (size_t)min(wave + 16 * i, nc - 1) * R + row;
    g.raw[i] = load_chunk<WT>(gu, o);
    g.sc[i] = gus[o];
  }
}
template <int WT, int MAXB>
__device__ __forceinline__ void gu_dots64(const GuRegs<WT>& g, int H, const uint16_t* xs, const float* xsum, int B,
                                          uint32_t mask, float (&acc)[MAXB], uint32_t magic) {
  const int wave = threadIdx.x >> 6, nc = H >> 5;
#pragma unroll
  for (int i = 0; i < F_GU_NB; i++) {
    const bool in = wave + 16 * i < nc;
    const int c = min(wave + 16 * i, nc - 1);
    uint32_t pr[16];
    qunpack32_m<WT>(g.raw[i], pr, magic);
    const float sc = in ? f16_to_f32(g.sc[i]) : 0.0f;
#pragma unroll
    for (int t = 0; t < MAXB; t++)
      if (t < B && ((mask >> t) & 1u))
        acc[t] = __builtin_fmaf(sc, qdot32_p<WT>(pr, xs + (size_t)t * H + 32 * c, xsum[t * nc + c]), acc[t]);
  }
}
// the 16 waves' row sums, then SwiGLU: token t's h (32 bf16) at s_hb + 32 t
template <int MAXB>
__device__ __forceinline__ void gu_swiglu64(const float (&acc)[MAXB], int B, uint32_t mask, float* s_red,
                                            uint16_t* s_hb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < MAXB; t++)
    if (t < B && ((mask >> t) & 1u)) s_red[(t * F_WAVES + wave) * 64 + lane] = acc[t];
  __syncthreads();
  const int t = threadIdx.x >> 5, j = threadIdx.x & 31;
  if (t < B && ((mask >> t) & 1u)) {
    const int gi = 32 * (j >> 4) + (j & 15), ui = gi + 16;
    float gs = 0.0f, us = 0.0f;
#pragma unroll
    for (int w = 0; w < F_WAVES; w++) {
      gs += s_red[(t * F_WAVES + w) * 64 + gi];
      us += s_red[(t * F_WAVES + w) * 64 + ui];
    }
    s_hb[32 * t + j] = f32_to_bf16(silu_f32(gs) * us);
  }
  __syncthreads();
}

template <int WT, int SWT, int MAXB>
__global__ __launch_bounds__(F_THREADS, 4) void k_decode1b(LayerDev L, const uint16_t* __restrict__ x,
                                                        uint16_t* __restrict__ y, int32_t* idx_out, float* gate_out,
                                                        DecodeWs ws, BatchGeo G) {
  static_assert(is_q<WT>(), "quantised routed experts");
  __shared__ __align__(16) uint16_t s_x[FB_XMAX];
  __shared__ __align__(16) float s_xsum[FB_XMAX / 32];
  __shared__ __align__(16) float s_red[FB_RED];  // reductions; the forwarder's top-k scratch before that
  __shared__ double s_rt[F_WAVES * MAXB * 4];  // router row sums: [wave][token][16-lane row]
  __shared__ int s_mark[64 * F_NV];
  __shared__ int s_nu;
  __shared__ int s_uexp[FB_SLOTS];
  __shared__ uint32_t s_umask[FB_SLOTS];
  __shared__ int s_sidx[FB_SLOTS];
  __shared__ int s_suid[FB_SLOTS];  // unique index of each slot's expert
  __shared__ float s_sgate[FB_SLOTS];
  __shared__ float s_ug[FB_SLOTS * FB_MAXB];  // gate of unique expert j for token t
  __shared__ uint32_t s_touch[F_NW];          // tokens each workgroup's partials cover
  __shared__ __align__(16) uint16_t s_hb[FB_MAXB * 32];
  __shared__ float s_hbs[FB_MAXB];
  const int H = L.H, I = L.I, B = G.B;
  const int b = blockIdx.x, tid = threadIdx.x, rank = start_rank(b);
  const uint32_t tag = ld_u32(my_counter(ws.sync)) + 1u;
  uint64_t* tl = reinterpret_cast<uint64_t*>(ws.logits);  // [B][E][2]
  uint64_t* res = ws.res_words + (size_t)(b % F_NX) * FB_RES_STRIDE;
  // [256][B][H] fp32 partials (untagged: read only after their producer's
  // done word)
  float* part = ws.part;
  uint64_t* xsw = ws.xsum_words;   // [8][B][H]
  uint64_t* pdone = ws.res_words + (size_t)F_NX * FB_RES_STRIDE;  // [256]: a workgroup's partials are in its XCD's L2
  const uint32_t allm = (1u << B) - 1u;
  const bool is_router = b < G.nR;
  const bool is_shared = b >= F_NX && b < F_NX + G.nSG;
  // the batch (B H / 8 16-byte pieces, two per thread) and the router rows
  // are loaded together, unconditionally (clamped)
  const int n8 = (B * H) >> 3;
  const uint4 v0 = reinterpret_cast<const uint4*>(x)[min(tid, n8 - 1)];
  const uint4 v1 = reinterpret_cast<const uint4*>(x)[min(tid + F_THREADS, n8 - 1)];
  RouterRegs rrg;
  router_issue(L, is_router, b, G.rr, rrg);
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int i = tid + F_THREADS * h;
    const uint4 v = h ? v1 : v0;
    if (i < n8) reinterpret_cast<uint4*>(s_x)[i] = v;
    // 32-element block sums: pieces 4b'..4b'+3 are lanes of one quad
    float sm = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
               ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
    sm += dpp_f32<DPP_XOR1>(sm);
    sm += dpp_f32<DPP_XOR2>(sm);
    if (i < n8 && (i & 3) == 0) s_xsum[i >> 2] = sm;
  }
  __syncthreads();
  if (is_router) router_finish_b<MAXB>(L, s_x, B, rrg, b, G.rr, tl, s_rt, tag);
  float pacc[MAXB][F_RPT];
#pragma unroll
  for (int t = 0; t < MAXB; t++)
#pragma unroll
    for (int n = 0; n < F_RPT; n++) pacc[t][n] = 0.0f;
  if (is_shared) {
    // shared unit su: intermediates 8su .. 8su+7, every token (while the
    // routing is made: after their routed units these workgroups were
    // last to finish, B = 3..8 1.2 - 3.1 us per call slower)
    constexpr int SW = (SWT == MOE_W_F32) ? MOE_W_F32 : MOE_W_BF16;
    const int su = b - F_NX, q = su >> 1, hf = su & 1;
    DownPre<SW> spre;
    gate_up_hb<SW, 16, MAXB>(L.sgu, nullptr, H, 2 * I, q, hf, s_x, nullptr, B, allm, s_red, s_hb,
                       [&] { down_prefetch<SW, 8>(L.sdn, nullptr, H, 16 * q + 8 * hf, spre); });
    constexpr int KCS = kchunk<SW>();
#pragma unroll
    for (int n = 0; n < F_RPT; n++) {
      const int row = tid + F_THREADS * n;
#pragma unroll
      for (int t = 0; t < MAXB; t++) {
        if (t < B) {
          float v = 0.0f;
          if constexpr (DownPlan<SW, 8>::PRE) {
            v = ddot<SW>(spre.r[n], s_hb + 32 * t, 0.0f);
          } else {
#pragma unroll
            for (int c = 0; c < 8 / KCS; c++)
              v = ddot<SW>(load_chunk<SW>(L.sdn, (size_t)((16 * q + 8 * hf) / KCS + c) * H + min(row, H - 1)),
                           s_hb + 32 * t + KCS * c, v);
          }
          pacc[t][n] += v;
        }
      }
    }
    __syncthreads();  // s_hb is reused
  }
  // the routing
  if (b < F_NX) {
    fwd_routing_b<MAXB>(L, tl, B, tag, ws.sync, G.wait_ticks, reinterpret_cast<uint8_t*>(s_red), s_mark, &s_nu, s_uexp,
                  s_umask, s_sidx, s_suid, s_sgate, res, idx_out, gate_out);
  } else {
    wait_routing_b(L, res, B, tag, ws.sync, G.wait_ticks, &s_nu, s_uexp, s_umask, s_sidx, s_suid, s_sgate);
  }
  const int nu = s_nu, nunits = nu * G.gpe;
  // gate of unique expert j for token t (0 where the token did not choose it)
  for (int i = tid; i < FB_SLOTS * FB_MAXB; i += F_THREADS) s_ug[i] = 0.0f;
  __syncthreads();
  if (tid < B * L.k) s_ug[s_suid[tid] * FB_MAXB + tid / L.k] = s_sgate[tid];
  for (int bb = tid; bb < F_NW; bb += F_THREADS) {
    uint32_t m = (bb >= F_NX && bb < F_NX + G.nSG) ? allm : 0u;
    for (int u = (bb - G.uoff + F_NW) % F_NW; u < nunits; u += F_NW) m |= s_umask[u / G.gpe];
    s_touch[bb] = m & allm;
  }
  __syncthreads();
  // routed units of this workgroup, u0, u0 + 256, ...: unit u + 256's loads
  // are issued as soon as unit u's registers are free (gate/up after its dot
  // products, down after its down products), so they are in flight while
  // unit u is finished. The last unit issues its own loads once more (the
  // lines are in the L2; a load under a branch would make the compiler wait
  // for it at once).
  const int u0 = (b - G.uoff + F_NW) % F_NW;
  if (u0 < nunits) {
    uint32_t magic = BF16_MAGIC2;
    asm volatile("" : "+v"(magic));
    GuRegs<WT> gr;
    DownPre<WT> pre;
    {
      const int j = u0 / G.gpe, q = u0 - j * G.gpe, e = s_uexp[j];
      gu_issue64<WT>(L.gu + (size_t)e * L.gu_stride, L.gu_s + (size_t)e * L.gu_s_stride, H, 2 * I, q, gr);
      down_prefetch<WT, 32>(L.dn + (size_t)e * L.dn_stride, L.dn_s + (size_t)e * L.dn_s_stride, H, 32 * q, pre);
    }
    for (int u = u0; u < nunits; u += F_NW) {
      const int j = u / G.gpe;
      const uint32_t mask = s_umask[j] & allm;
      const int un = (u + F_NW < nunits) ? u + F_NW : u;
      const int jn = un / G.gpe, qn = un - jn * G.gpe, en = s_uexp[jn];
      float acc[MAXB];
#pragma unroll
      for (int t = 0; t < MAXB; t++) acc[t] = 0.0f;
      gu_dots64<WT, MAXB>(gr, H, s_x, s_xsum, B, mask, acc, magic);
      gu_issue64<WT>(L.gu + (size_t)en * L.gu_stride, L.gu_s + (size_t)en * L.gu_s_stride, H, 2 * I, qn, gr);
      gu_swiglu64<MAXB>(acc, B, mask, s_red, s_hb);
      // each token's block sum of its 32 h values (32 lanes, fixed order)
      {
        // lanes of one 32-lane half: sum16 over each row of 16, then the two rows
        const int t = tid >> 5;
        const bool act = tid < 32 * MAXB && t < B && ((mask >> t) & 1u);
        float v = act ? bf16_to_f32(s_hb[min(tid, 32 * MAXB - 1)]) : 0.0f;
        v = sum16_f32(v);
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16 (bit-mode swizzle)
        if (act && (tid & 31) == 0) s_hbs[t] = v;
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < F_RPT; n++) {
        uint32_t pr[16];
        qunpack32_m<WT>(pre.r[n], pr, magic);
        const float sc = f16_to_f32(pre.s[n]);
#pragma unroll
        for (int t = 0; t < MAXB; t++)
          if (t < B && ((mask >> t) & 1u))
            pacc[t][n] = __builtin_fmaf(sc * qdot32_p<WT>(pr, s_hb + 32 * t, s_hbs[t]), s_ug[j * FB_MAXB + t], pacc[t][n]);
      }
      down_prefetch<WT, 32>(L.dn + (size_t)en * L.dn_stride, L.dn_s + (size_t)en * L.dn_s_stride, H, 32 * qn, pre);
      __syncthreads();  // s_red, s_hb and s_hbs are reused by the next unit
    }
  }
  // this workgroup's partials of the tokens it touched, into its XCD's L2
  {
    const uint32_t mine = s_touch[b];
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < B && ((mine >> t) & 1u)) {
#pragma unroll
        for (int n = 0; n < F_RPT; n++) {
          const int row = tid + F_THREADS * n;
          if (row < H) part[((size_t)b * B + t) * H + row] = pacc[t][n];
        }
      }
    }
    // every partial has reached the XCD's L2 (vmcnt counts stores until the
    // L2 acknowledges them) before any wave passes the barrier, and so before
    // the done word is stored: a reader that sees the done word finds them
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) st_word_xcd(pdone + b, 0u, tag);
  }
  // XCD-level sums: workgroup jx of XCD x sums rows r0 .. r0 + H/32 - 1 of
  // every token over the producers of its XCD (workgroups x + 8 j', j' in
  // order) that touched the token
  {
    const int xx = b % F_NX, jx = b / F_NX;
    const int nrow = H / F_PX, r0 = jx * nrow;
    const int rr = tid & 63, g = tid >> 6;
    const int row = r0 + min(rr, nrow - 1);
    const int pb0 = xx + F_NX * g, pb1 = xx + F_NX * (g + 16);
    const uint32_t tm0 = s_touch[pb0], tm1 = s_touch[pb1];
    // each wave waits for its own two producers' done words (wave g:
    // workgroups xx + 8 g and xx + 8 (g + 16)) and loads a producer's
    // partials as soon as that producer is done, while the XCD's later
    // producers still run: the early partials are read while they are still
    // in the L2 (waiting for all 32 first left them to be read back from
    // memory at the end, up to 4 MB per XCD at B = 8)
    // (both done words are loaded up front: when both producers are already
    // done, both producers' partials are requested back to back)
    const uint64_t* dw0 = pdone + pb0;
    const uint64_t* dw1 = pdone + pb1;
    uint64_t d0 = ld_word_coherent(dw0), d1 = ld_word_coherent(dw1);
    const bool nd0 = (tm0 & allm) != 0u, nd1 = (tm1 & allm) != 0u;  // wave-uniform
    const uint64_t c0 = wall_clock64();
    if (__builtin_amdgcn_ballot_w64(nd0 && !tag_ok(d0, tag)) != 0) {
      int it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(2);
        const uint64_t n0 = ld_word_coherent(dw0), n1 = ld_word_coherent(dw1);
        d0 = tag_ok(d0, tag) ? d0 : n0;
        d1 = tag_ok(d1, tag) ? d1 : n1;
        if (__builtin_amdgcn_ballot_w64(!tag_ok(d0, tag)) == 0) break;
        if ((++it & 15) == 0 && wall_clock64() - c0 > G.wait_ticks) {
          if ((tid & 63) == 0) flag_error(ws.sync, 4u);
          break;
        }
      }
    }
    float w0[MAXB], w1[MAXB];
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      const int tt = min(t, B - 1);
      w0[t] = ld_f32_coherent(part + ((size_t)pb0 * B + tt) * H + row);  // unconditional, clamped
    }
    if (__builtin_amdgcn_ballot_w64(nd1 && !tag_ok(d1, tag)) != 0) {
      int it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(2);
        d1 = ld_word_coherent(dw1);
        if (__builtin_amdgcn_ballot_w64(!tag_ok(d1, tag)) == 0) break;
        if ((++it & 15) == 0 && wall_clock64() - c0 > G.wait_ticks) {
          if ((tid & 63) == 0) flag_error(ws.sync, 4u);
          break;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      const int tt = min(t, B - 1);
      w1[t] = ld_f32_coherent(part + ((size_t)pb1 * B + tt) * H + row);
    }
    auto need0 = [&](int t) { return t < B && ((tm0 >> t) & 1u); };
    auto need1 = [&](int t) { return t < B && ((tm1 >> t) & 1u); };
#pragma unroll
    for (int t = 0; t < MAXB; t++) {
      if (t < B) {
        float a = need0(t) ? w0[t] : 0.0f;
        a += need1(t) ? w1[t] : 0.0f;
        s_red[(t * F_WAVES + g) * 64 + rr] = a;
      }
    }
    __syncthreads();
    if (tid < 64 * B) {
      const int t = tid >> 6, r2 = tid & 63;
      if (r2 < nrow) {
        float sm = 0.0f;
#pragma unroll
        for (int q = 0; q < F_WAVES; q++) sm += s_red[(t * F_WAVES + q) * 64 + r2];
        st_word(xsw + ((size_t)xx * B + t) * H + r0 + r2, __float_as_uint(sm), tag);
      }
    }
  }
  // final: rows row0 .. row0 + nr - 1 of every token; wave t takes token t,
  // lane l row l % 8 and XCD l / 8, the XCDs added in order
  {
    const int row0 = rank * H / F_NW, nr = (rank + 1) * H / F_NW - row0;
    const int wave = tid >> 6, lane = tid & 63;
    if (wave < B && nr > 0) {
      const int r = lane & 7, qx = lane >> 3;
      const bool use = r < nr;
      const uint64_t* pw = xsw + ((size_t)qx * B + wave) * H + row0 + min(r, nr - 1);
      uint64_t w = ld_word_coherent(pw);
      if (__builtin_amdgcn_ballot_w64(use && !tag_ok(w, tag)) != 0) {
        const uint64_t c0 = wall_clock64();
        int it = 0;
        while (true) {
          __builtin_amdgcn_s_sleep(1);
          const uint64_t nw = ld_word_coherent(pw);
          w = tag_ok(w, tag) ? w : nw;
          if (__builtin_amdgcn_ballot_w64(use && !tag_ok(w, tag)) == 0) break;
          if ((++it & 15) == 0 && wall_clock64() - c0 > G.wait_ticks) {
            if (lane == 0) flag_error(ws.sync, 8u);
            break;
          }
        }
      }
      const float v = use ? __uint_as_float((uint32_t)w) : 0.0f;
      float t = v;
#pragma unroll
      for (int qq = 1; qq < F_NX; qq++) t += __shfl(v, r + 8 * qq, 64);
      if (lane < nr) y[(size_t)wave * H + row0 + lane] = f32_to_bf16(t);
    }
  }
  finish(ws.sync, tag);
}

size_t decode1b_part_words(int H, int B) { return (size_t)F_NW * B * H; }
size_t decode1b_xsum_words(int H, int B) { return (size_t)F_NX * B * H; }
size_t decode1b_res_words() { return (size_t)F_NX * FB_RES_STRIDE + F_NW; }  // routing words, then done words

// Batch widths compiled (a call's batch is padded to the next one): every
// token slot costs router sums, unit loops and partial loads whether the call
// fills it or not. Q4: 2, 3, 4, 5, 8; Q3: 2, 3, 4, 8 (its width-5 build
// spills to scratch).
template <int WT, int MAXB>
static bool no_scratch_b() {
  return no_scratch(k_decode1b<WT, MOE_W_NONE, MAXB>) && no_scratch(k_decode1b<WT, MOE_W_F32, MAXB>) &&
         no_scratch(k_decode1b<WT, MOE_W_BF16, MAXB>);
}
static bool decode1b_no_scratch() {
  static const bool ok = no_scratch_b<MOE_W_Q4, 2>() && no_scratch_b<MOE_W_Q4, 3>() && no_scratch_b<MOE_W_Q4, 4>() &&
                         no_scratch_b<MOE_W_Q4, 5>() && no_scratch_b<MOE_W_Q4, 8>() && no_scratch_b<MOE_W_Q3, 2>() &&
                         no_scratch_b<MOE_W_Q3, 3>() && no_scratch_b<MOE_W_Q3, 4>() && no_scratch_b<MOE_W_Q3, 8>();
  return ok;
}

bool decode1b_fits(int wt, int E, int H, int I, int k, bool has_shared, int B) {
  // quantised routed experts; the batch-1 limits on E, H, I and k; B k <= 128
  // slots; the shared units and the forwarders within the grid
  const int nSG = has_shared ? I / 8 : 0;
  return (wt == MOE_W_Q4 || wt == MOE_W_Q3) && B >= 2 && B <= FB_MAXB && B * H <= FB_XMAX &&
         E <= 64 * F_NV && E <= F_NW * F_RRMAX && H <= F_HMAX && H % 32 == 0 && I <= 1024 && k <= 16 &&
         F_NX + nSG <= F_NW && F_NW <= decode1_capacity() && decode1b_no_scratch();
}

template <int WT, int SWT, int MAXB>
static hipError_t launch_fused_bt(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out,
                                  float* gate_out, const DecodeWs& ws, hipStream_t st) {
  BatchGeo G;
  G.B = B;
  G.rr = L.E > F_NW ? 2 : 1;
  G.nR = (L.E + G.rr - 1) / G.rr;
  G.nSG = (SWT == MOE_W_NONE) ? 0 : L.I / 8;
  G.gpe = L.I / 32;
  G.uoff = F_NX + G.nSG;
  G.wait_ticks = g_wait_ticks;
  return launch_k(KC_DEC_FUSED, k_decode1b<WT, SWT, MAXB>, dim3(F_NW), dim3(F_THREADS), 0, st, L, x, y, idx_out,
                  gate_out, ws, G);
}

template <int WT, int MAXB>
static hipError_t launch_fused_bs(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                                  const DecodeWs& ws, hipStream_t st) {
  if (L.swt == MOE_W_NONE) return launch_fused_bt<WT, MOE_W_NONE, MAXB>(L, x, B, y, io, go, ws, st);
  if (L.swt == MOE_W_F32) return launch_fused_bt<WT, MOE_W_F32, MAXB>(L, x, B, y, io, go, ws, st);
  return launch_fused_bt<WT, MOE_W_BF16, MAXB>(L, x, B, y, io, go, ws, st);
}
template <int WT>
static hipError_t launch_fused_bw(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* io, float* go,
                                  const DecodeWs& ws, hipStream_t st) {
  if (B == 2) return launch_fused_bs<WT, 2>(L, x, B, y, io, go, ws, st);
  if (B == 3) return launch_fused_bs<WT, 3>(L, x, B, y, io, go, ws, st);
  if (B == 4) return launch_fused_bs<WT, 4>(L, x, B, y, io, go, ws, st);
  if constexpr (WT == MOE_W_Q4)
    if (B == 5) return launch_fused_bs<WT, 5>(L, x, B, y, io, go, ws, st);
  return launch_fused_bs<WT, 8>(L, x, B, y, io, go, ws, st);
}

hipError_t launch_decode_fused_b(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out,
                                 float* gate_out, const DecodeWs& ws, hipStream_t st) {
  if (L.wt == MOE_W_Q4) return launch_fused_bw<MOE_W_Q4>(L, x, B, y, idx_out, gate_out, ws, st);
  return launch_fused_bw<MOE_W_Q3>(L, x, B, y, idx_out, gate_out, ws, st);
}

}  // namespace moe
