// Host/device shared parameter blocks and launch declarations (internal).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Kernel classes for the optional timer.
enum KernelClass {
  KC_DEC_FUSED = 0,          // batch-1 decode, one kernel
  KC_DEC_ROUTER_SHARED,      // router logits + the whole shared expert
  KC_DEC_GATE_UP,            // routed experts (gate/up, SwiGLU, partial down)
  KC_DEC_DOWN,               // sum of the partial down products
  KC_PF_ROUTER,
  KC_PF_TOPK,
  KC_PF_COUNT,
  KC_PF_SCAN,
  KC_PF_SCATTER,
  KC_PF_GATE_UP,
  KC_PF_DOWN,
  KC_PF_SHARED_GATE_UP,
  KC_PF_SHARED_DOWN,
  KC_PF_COMBINE,
  KC_NORM,
  KC_RESIDUAL,
  KC_FILL,
  KC_DEC_ROUTE,              // top-k of a batch and its unique experts (B > 1 path)
  KC_PF_RSPLIT,              // router weights split into two bf16 halves + row norms
  KC_COUNT
};

struct LayerDev {
  int32_t H, I, E, k;
  const float* router_w;
  const float* router_b;
  int32_t wt;
  const uint8_t* gu;
  const uint16_t* gu_s;
  const uint8_t* dn;
  const uint16_t* dn_s;
  int32_t swt;
  const uint8_t* sgu;
  const uint8_t* sdn;
  size_t gu_stride;    // bytes per expert (fused gate/up values)
  size_t gu_s_stride;  // scales per expert
  size_t dn_stride;
  size_t dn_s_stride;
};

// Decode workspace (all device pointers inside the caller's workspace).
struct DecodeWs {
  uint32_t* sync;  // counts and epoch of the one-kernel path (counts zero between calls)
  double* logits;  // four-kernel path: [B][E] fp64; one-kernel path: rotating slots of [E][2] tagged words
  float* part;     // four-kernel path: [B*k*(I/16) + B*(I/8)][H] partial down products;
                   // batched one-kernel path: [256][B][H] per-workgroup partials (untagged)
  uint64_t* part_words;  // one-kernel path: [producers][H] tagged partial down products (fp32 bits), read within each XCD
  uint64_t* xsum_words;  // one-kernel path: [8][H] tagged per-XCD sums of the partials
  uint32_t* ctr;         // one-kernel path: router counters, rotating slots x XCD groups, one 128-byte line each
  uint64_t* res_words;   // batched one-kernel path: [8][512] tagged routing words per XCD
  int32_t* route;        // four-kernel path: the batch's routing (count, idx, gates, unique experts, masks)
  uint16_t* zb;          // [B][H] bf16: z of a stack layer taken as separate kernels
  uint16_t* yb;          // [B][H] bf16: its y
};

// Prefill workspace.
struct PrefillWs {
  double* logits;     // [T][E] (approximate fp32 logits in the first half)
  uint16_t* rsplit;   // [2][E][H] router weights as bf16 hi, then lo
  double* wnorm;      // [E] router row norms
  int32_t* idx;       // [T][k]
  float* gates;       // [T][k]
  int32_t* blk_counts;// [nblk][E]
  int32_t* blk_base;  // [nblk][E]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* tile_start;// [E+1] routed GEMM M-tiles per expert, prefix summed
  int32_t* tile_info; // [T*k/PF_BM + E][PF_TILE_INFO] per M tile: expert, first tile, tiles, row offset, rows
  int32_t* perm;      // [T*k] sorted position -> slot
  int32_t* inv;       // [T*k] slot -> sorted position
  uint16_t* h;        // [T*k][I] bf16, sorted order
  uint16_t* hs;       // [T][I] bf16, shared expert
  uint16_t* Y;        // [T*k][H] bf16, sorted order, un-gated expert outputs
  uint16_t* Ys;       // [T][H] bf16, shared expert output
};

// Launch wrappers (return hipError_t of the launch).
size_t decode_lds_b(int wt, int B, int H, int E, int k);  // LDS bytes of the routed-expert kernel
size_t decode1_lds(int H, int I, int k, bool has_shared);  // LDS bytes of the one-kernel batch-1 path
size_t decode1_logit_words(int E);  // rotating slots x XCD-group replicas x [E][2] tagged words
size_t decode1_part_words(int H, int I, int k, bool has_shared);
size_t decode1_xsum_words(int H);
size_t decode1_counter_words();
bool decode1_fits(int E, int H, int I, int k, bool has_shared);  // shape handled by the one-kernel path
// batched one-kernel path (B = 2..8): [256][B][H] fp32 partials, [8][B][H] XCD sums, [8][512] routing words
bool decode1b_fits(int wt, int E, int H, int I, int k, bool has_shared, int B);
size_t decode1b_part_words(int H, int B);
size_t decode1b_xsum_words(int H, int B);
size_t decode1b_res_words();
void decode1_set_wait_ticks(uint64_t ticks);  // bound of the one-kernel path's waits (0: the default)
// One layer of a pre-norm residual stack, in place on the residual stream h:
// z = RMSNorm(h), y = MoE(z), h = bf16(h + y); z_out / y_out optional copies.
struct StackIo {
  uint16_t* h;      // [H] bf16 residual stream (NULL: plain decode, x -> y)
  uint16_t* z_out;  // [H] or NULL
  uint16_t* y_out;  // [H] or NULL
  float eps;
};
hipError_t launch_decode_fused(const LayerDev& L, const uint16_t* x, uint16_t* y, int32_t* idx_out,
                               float* gate_out, const DecodeWs& ws, hipStream_t st, const StackIo* stack = nullptr);
hipError_t launch_decode_fused_b(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out,
                                 float* gate_out, const DecodeWs& ws, hipStream_t st);
hipError_t launch_decode(const LayerDev& L, const uint16_t* x, int B, uint16_t* y, int32_t* idx_out,
                         float* gate_out, const DecodeWs& ws, hipStream_t st);
hipError_t launch_stack_decode(const LayerDev& L, uint16_t* h, int B, float eps, uint16_t* z_out, uint16_t* y_out,
                               int32_t* idx_out, float* gate_out, const DecodeWs& ws, hipStream_t st);
hipError_t launch_route(const LayerDev& L, const uint16_t* x, int T, int32_t* idx_out, float* gate_out,
                        int32_t* counts_out, const PrefillWs& ws, hipStream_t st);
hipError_t launch_prefill(const LayerDev& L, const uint16_t* x, int T, uint16_t* y, int32_t* idx_out,
                          float* gate_out, const PrefillWs& ws, hipStream_t st);
hipError_t launch_rmsnorm(const uint16_t* h, uint16_t* z, int T, int H, float eps, hipStream_t st);
hipError_t launch_residual(uint16_t* h, const uint16_t* y, int T, int H, hipStream_t st);
hipError_t launch_fill(void* p, size_t bytes, hipStream_t st);

// Prefill tiling constants shared by host sizing and kernels.
constexpr int PF_BM = 96;           // max rows (tokens) per grouped-GEMM tile
constexpr int PF_TILE_INFO = 8;     // int32 words per M-tile record (5 used, 32-byte aligned)
constexpr int PF_TOK_PER_BLK = 256; // tokens per histogram block

// Timer hooks (api.cpp). When the timer is on, a launch carries a start and
// a stop event in its own dispatch packet, so the measured interval is the
// kernel's execution, not the gap between host-side records.
bool timer_events(int kc, hipEvent_t* start, hipEvent_t* stop);
void timer_commit(int kc, hipEvent_t start, hipEvent_t stop);

template <typename F, typename... Args>
hipError_t launch_k(int kc, F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timer_events(kc, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0u, args...);
    timer_commit(kc, e0, e1);
  } else {
    kernel<<<grid, block, lds, st>>>(args...);
  }
  return hipPeekAtLastError();  // sticky: the caller's hipGetLastError() reports it
}

}  // namespace moe
