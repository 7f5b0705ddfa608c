// C ABI: argument validation, workspace layout, host packing, diagnostics.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

bool is_expert_wt(int32_t wt) { return wt == MOE_W_F32 || wt == MOE_W_BF16 || wt == MOE_W_Q4 || wt == MOE_W_Q3; }
bool is_quant(int32_t wt) { return wt == MOE_W_Q4 || wt == MOE_W_Q3; }

// bytes per 16-byte-class chunk and elements per chunk
int chunk_bytes(int32_t wt) { return wt == MOE_W_Q3 ? 12 : 16; }
int chunk_elems(int32_t wt) { return wt == MOE_W_F32 ? 4 : wt == MOE_W_BF16 ? 8 : 32; }

moe_status check_shape(const moe_layer* L) {
  if (!L) return fail(MOE_ERR_NULL, "layer is NULL");
  if (L->hidden < 32 || L->hidden > 8192 || L->hidden % 32)
    return fail(MOE_ERR_SHAPE, "hidden=%d must be a multiple of 32 in [32, 8192]", L->hidden);
  if (L->inter < 32 || L->inter > 4096 || L->inter % 32)
    return fail(MOE_ERR_SHAPE, "inter=%d must be a multiple of 32 in [32, 4096]", L->inter);
  if (L->n_experts < 1 || L->n_experts > 1024) return fail(MOE_ERR_SHAPE, "n_experts=%d not in [1, 1024]", L->n_experts);
  if (L->top_k < 1 || L->top_k > 16 || L->top_k > L->n_experts)
    return fail(MOE_ERR_SHAPE, "top_k=%d not in [1, min(16, n_experts)]", L->top_k);
  if (!is_expert_wt(L->expert_wtype)) return fail(MOE_ERR_DTYPE, "expert_wtype=%d unsupported", L->expert_wtype);
  if (L->shared_wtype != MOE_W_NONE && L->shared_wtype != MOE_W_F32 && L->shared_wtype != MOE_W_BF16)
    return fail(MOE_ERR_DTYPE, "shared_wtype=%d unsupported (F32, BF16 or NONE)", L->shared_wtype);
  return MOE_OK;
}

moe_status check_layer(const moe_layer* L) {
  moe_status st = check_shape(L);
  if (st != MOE_OK) return st;
  if (!L->router_w) return fail(MOE_ERR_NULL, "router_w is NULL");
  if (!L->gate_up || !L->down) return fail(MOE_ERR_NULL, "expert weights are NULL");
  if (is_quant(L->expert_wtype) && (!L->gate_up_scales || !L->down_scales))
    return fail(MOE_ERR_NULL, "quantised experts need gate_up_scales and down_scales");
  if (L->shared_wtype != MOE_W_NONE && (!L->shared_gate_up || !L->shared_down))
    return fail(MOE_ERR_NULL, "shared expert weights are NULL");
  const void* ptrs[] = {L->router_w, L->router_bias, L->gate_up, L->gate_up_scales, L->down, L->down_scales,
                        L->shared_gate_up, L->shared_down};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MOE_ERR_ALIGN, "a layer pointer is not 16-byte aligned");
  return MOE_OK;
}

moe::LayerDev to_dev(const moe_layer* L) {
  moe::LayerDev d{};
  d.H = L->hidden; d.I = L->inter; d.E = L->n_experts; d.k = L->top_k;
  d.router_w = L->router_w; d.router_b = L->router_bias;
  d.wt = L->expert_wtype;
  d.gu = static_cast<const uint8_t*>(L->gate_up); d.gu_s = L->gate_up_scales;
  d.dn = static_cast<const uint8_t*>(L->down); d.dn_s = L->down_scales;
  d.swt = L->shared_wtype;
  d.sgu = static_cast<const uint8_t*>(L->shared_gate_up);
  d.sdn = static_cast<const uint8_t*>(L->shared_down);
  d.gu_stride = moe_matrix_bytes(d.wt, 2 * d.I, d.H);
  d.gu_s_stride = moe_matrix_scales(d.wt, 2 * d.I, d.H);
  d.dn_stride = moe_matrix_bytes(d.wt, d.H, d.I);
  d.dn_s_stride = moe_matrix_scales(d.wt, d.H, d.I);
  return d;
}

constexpr size_t DECODE_SYNC_BYTES = 4096;  // counters at the start of a decode workspace (word 0: error bits)

// Workspace carving. ptr == nullptr only sizes.
size_t carve_decode(const moe_layer* L, int B, uint8_t* base, moe::DecodeWs* ws) {
  const size_t E = L->n_experts, k = L->top_k, I = L->inter;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  };
  moe::DecodeWs w{};
  w.sync = reinterpret_cast<uint32_t*>(take(DECODE_SYNC_BYTES));
  const bool has_s = L->shared_wtype != MOE_W_NONE;
  const bool one_kernel = B == 1 && moe::decode1_fits(L->n_experts, L->hidden, L->inter, L->top_k, has_s);
  const bool one_kernel_b =
      B > 1 && moe::decode1b_fits(L->expert_wtype, L->n_experts, L->hidden, L->inter, L->top_k, has_s, B);
  // logits: [B][E] fp64 (four kernels), rotating slots of per-XCD-group [E] x 16 B tagged words (one kernel,
  // batch 1) or [B][E] x 16 B tagged words (one kernel, batched)
  w.logits = reinterpret_cast<double*>(take(one_kernel     ? 8 * moe::decode1_logit_words((int)E)
                                             : one_kernel_b ? (size_t)B * E * 16
                                                            : (size_t)E * 64));
  if (one_kernel_b) {
    w.part = reinterpret_cast<float*>(take(4 * moe::decode1b_part_words(L->hidden, B)));
    w.xsum_words = reinterpret_cast<uint64_t*>(take(8 * moe::decode1b_xsum_words(L->hidden, B)));
    w.res_words = reinterpret_cast<uint64_t*>(take(8 * moe::decode1b_res_words()));
  } else if (one_kernel) {
    w.part_words = reinterpret_cast<uint64_t*>(take(8 * moe::decode1_part_words(L->hidden, L->inter, L->top_k, has_s)));
    w.xsum_words = reinterpret_cast<uint64_t*>(take(8 * moe::decode1_xsum_words(L->hidden)));
    w.ctr = reinterpret_cast<uint32_t*>(take(4 * moe::decode1_counter_words()));
  } else {
    w.part = reinterpret_cast<float*>(take((size_t)B * (k * (I / 16) + I / 8) * L->hidden * 4));
    w.route = reinterpret_cast<int32_t*>(take((4 + 4 * 8 * 16) * 4));
  }
  // z and y of a stack layer run as separate kernels (moe_stack_decode_layer)
  w.zb = reinterpret_cast<uint16_t*>(take((size_t)B * L->hidden * 2));
  w.yb = reinterpret_cast<uint16_t*>(take((size_t)B * L->hidden * 2));
  if (ws) *ws = w;
  return off;
}

size_t carve_prefill(const moe_layer* L, int T, uint8_t* base, moe::PrefillWs* ws) {
  const size_t E = L->n_experts, k = L->top_k, I = L->inter, H = L->hidden;
  const size_t nblk = ((size_t)T + moe::PF_TOK_PER_BLK - 1) / moe::PF_TOK_PER_BLK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  };
  moe::PrefillWs w{};
  w.logits = reinterpret_cast<double*>(take((size_t)T * E * 8));
  w.rsplit = reinterpret_cast<uint16_t*>(take(E * H * 2 * 2));
  w.wnorm = reinterpret_cast<double*>(take(E * 8));
  w.idx = reinterpret_cast<int32_t*>(take((size_t)T * k * 4));
  w.gates = reinterpret_cast<float*>(take((size_t)T * k * 4));
  w.blk_counts = reinterpret_cast<int32_t*>(take(nblk * E * 4));
  w.blk_base = reinterpret_cast<int32_t*>(take(nblk * E * 4));
  w.counts = reinterpret_cast<int32_t*>(take(E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.tile_start = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.tile_info = reinterpret_cast<int32_t*>(take(((size_t)T * k / moe::PF_BM + 1 + E) * moe::PF_TILE_INFO * 4));
  w.perm = reinterpret_cast<int32_t*>(take((size_t)T * k * 4));
  w.inv = reinterpret_cast<int32_t*>(take((size_t)T * k * 4));
  w.h = reinterpret_cast<uint16_t*>(take((size_t)T * k * I * 2));
  w.hs = reinterpret_cast<uint16_t*>(take((size_t)T * I * 2));
  w.Y = reinterpret_cast<uint16_t*>(take((size_t)T * k * H * 2));
  w.Ys = reinterpret_cast<uint16_t*>(take((size_t)T * H * 2));
  if (ws) *ws = w;
  return off;
}

constexpr int PREFILL_MAX_TOKENS = 1 << 20;

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// Kernel timer
// ---------------------------------------------------------------------------
struct Pending {
  int kc;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timer_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
int64_t g_launches[moe::KC_COUNT];
double g_ms[moe::KC_COUNT];

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_locked() {
  for (auto& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_launches[p.kc]++;
      g_ms[p.kc] += ms;
    }
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
}

const char* const kKernelNames[moe::KC_COUNT] = {
    "dec_fused",         "dec_router_shared", "dec_routed", "dec_reduce",         "pf_router",         "pf_topk",
    "pf_count",          "pf_scan",     "pf_scatter",       "pf_gate_up",        "pf_down",
    "pf_shared_gate_up", "pf_shared_down", "pf_combine",    "rmsnorm",           "residual_add",
    "fill",              "dec_route",       "pf_rsplit"};

}  // namespace

namespace moe {
bool timer_events(int kc, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_timer_on) return false;
  std::lock_guard<std::mutex> lk(g_tmu);
  (void)kc;
  hipEvent_t a = get_event(), b = get_event();
  if (!a || !b) {
    if (a) g_pool.push_back(a);
    if (b) g_pool.push_back(b);
    return false;
  }
  *start = a;
  *stop = b;
  return true;
}
void timer_commit(int kc, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_pending.push_back({kc, start, stop});
  if (g_pending.size() > 4096) drain_locked();
}
}  // namespace moe

extern "C" {

size_t moe_matrix_bytes(int32_t wt, int32_t rows, int32_t K) {
  if (!is_expert_wt(wt) || rows <= 0 || K <= 0 || K % 32) return 0;
  return (size_t)(K / chunk_elems(wt)) * (size_t)rows * chunk_bytes(wt);
}

size_t moe_matrix_scales(int32_t wt, int32_t rows, int32_t K) {
  if (!is_quant(wt) || rows <= 0 || K <= 0 || K % 32) return 0;
  return (size_t)(K / 32) * (size_t)rows;
}

size_t moe_workspace_bytes(const moe_layer* layer, int32_t max_tokens, int32_t mode) {
  if (check_shape(layer) != MOE_OK) return 0;
  if (mode == 0) {
    if (max_tokens < 1 || max_tokens > MOE_DECODE_MAX_TOKENS) return 0;
    size_t m = 0;
    for (int b = 1; b <= max_tokens; b++) {
      const size_t n = carve_decode(layer, b, nullptr, nullptr);
      m = n > m ? n : m;
    }
    return m;
  }
  if (mode == 1) {
    if (max_tokens < 1 || max_tokens > PREFILL_MAX_TOKENS) return 0;
    return carve_prefill(layer, max_tokens, nullptr, nullptr);
  }
  return 0;
}

moe_status moe_route(const moe_layer* layer, const void* x, int32_t T, int32_t* topk_idx, float* topk_gate,
                     int32_t* expert_counts, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !topk_idx || !topk_gate || !ws) return fail(MOE_ERR_NULL, "x, topk_idx, topk_gate and ws are required");
  if (T < 1 || T > PREFILL_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "T=%d not in [1, %d]", T, PREFILL_MAX_TOKENS);
  if (!aligned16(x) || !aligned16(ws)) return fail(MOE_ERR_ALIGN, "x and ws must be 16-byte aligned");
  const size_t need = carve_prefill(layer, T, nullptr, nullptr);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  moe::PrefillWs w;
  carve_prefill(layer, T, static_cast<uint8_t*>(ws), &w);
  return hip_status(moe::launch_route(to_dev(layer), static_cast<const uint16_t*>(x), T, topk_idx, topk_gate,
                                      expert_counts, w, stream),
                    "moe_route launch");
}

moe_status moe_forward_decode(const moe_layer* layer, const void* x, int32_t B, void* y, int32_t* topk_idx,
                              float* topk_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws) return fail(MOE_ERR_NULL, "x, y and ws are required");
  if (B < 1 || B > MOE_DECODE_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "B=%d not in [1, %d]", B, MOE_DECODE_MAX_TOKENS);
  if ((int64_t)B * layer->hidden > 8 * 2048)
    return fail(MOE_ERR_SHAPE, "B*H=%d exceeds the decode staging limit %d", B * layer->hidden, 8 * 2048);
  const bool has_s = layer->shared_wtype != MOE_W_NONE;
  const bool one_kernel =
      (B == 1 && moe::decode1_fits(layer->n_experts, layer->hidden, layer->inter, layer->top_k, has_s)) ||
      (B > 1 && moe::decode1b_fits(layer->expert_wtype, layer->n_experts, layer->hidden, layer->inter, layer->top_k,
                                   has_s, B));
  if (!one_kernel && moe::decode_lds_b(layer->expert_wtype, B, layer->hidden, layer->n_experts, layer->top_k) > 65536)
    return fail(MOE_ERR_SHAPE, "B=%d with H=%d, E=%d, k=%d needs more than 64 KiB of LDS", B, layer->hidden,
                layer->n_experts, layer->top_k);
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return fail(MOE_ERR_ALIGN, "x, y and ws must be 16-byte aligned");
  const size_t need = carve_decode(layer, B, nullptr, nullptr);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  moe::DecodeWs w;
  carve_decode(layer, B, static_cast<uint8_t*>(ws), &w);
  return hip_status(moe::launch_decode(to_dev(layer), static_cast<const uint16_t*>(x), B, static_cast<uint16_t*>(y),
                                       topk_idx, topk_gate, w, stream),
                    "moe_forward_decode launch");
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the workspace is a static device array
// of the library (one per GPU, held until the process ends). Its device
// address is looked up once per device and used everywhere host code needs
// the array's memory; the array's name itself is only a host-side stand-in.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

struct ScratchDev {
  void* ptr = nullptr;  // device address of `scratch` on this device (nullptr: not set up yet)
};
static std::mutex g_scratch_mu;
static ScratchDev g_scratch[64];

// Device address of the array on the current device; on the first call per
// device also zero it (the decode workspace contract) and wait for that.
static moe_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev].ptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_status(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(MOE_ERR_SHAPE, "the first moe_forward_decode_noalloc call on a device must not be under graph "
                                 "capture (it sets up and zeroes the device's scratch array)");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    e = moe::launch_fill(p, MOE_NOALLOC_SCRATCH_BYTES, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e, "zeroing the scratch array");
    g_scratch[dev].ptr = p;
  }
  *out = g_scratch[dev].ptr;
  return MOE_OK;
}

moe_status moe_forward_decode_noalloc(const moe_layer* layer, const void* x, int32_t B, void* y, int32_t* topk_idx,
                                      float* topk_gate, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y) return fail(MOE_ERR_NULL, "x and y are required");
  if (B < 1 || B > MOE_DECODE_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "B=%d not in [1, %d]", B, MOE_DECODE_MAX_TOKENS);
  const size_t need = carve_decode(layer, B, nullptr, nullptr);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "this layer and B=%d need %zu workspace bytes, more than the %u bytes of the "
                                   "library's scratch array; use moe_forward_decode with a workspace",
                B, need, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(stream, &ws);
  if (st != MOE_OK) return st;
  return moe_forward_decode(layer, x, B, y, topk_idx, topk_gate, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_stack_decode_layer(const moe_layer* layer, void* h, int32_t B, float eps, void* z_out, void* y_out,
                                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!h || !ws) return fail(MOE_ERR_NULL, "h and ws are required");
  if (B < 1 || B > MOE_DECODE_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "B=%d not in [1, %d]", B, MOE_DECODE_MAX_TOKENS);
  if ((int64_t)B * layer->hidden > 8 * 2048)
    return fail(MOE_ERR_SHAPE, "B*H=%d exceeds the decode staging limit %d", B * layer->hidden, 8 * 2048);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_SHAPE, "eps must be >= 0");
  const bool has_s = layer->shared_wtype != MOE_W_NONE;
  const bool one_kernel =
      (B == 1 && moe::decode1_fits(layer->n_experts, layer->hidden, layer->inter, layer->top_k, has_s)) ||
      (B > 1 && moe::decode1b_fits(layer->expert_wtype, layer->n_experts, layer->hidden, layer->inter, layer->top_k,
                                   has_s, B));
  if (!one_kernel && moe::decode_lds_b(layer->expert_wtype, B, layer->hidden, layer->n_experts, layer->top_k) > 65536)
    return fail(MOE_ERR_SHAPE, "B=%d with H=%d, E=%d, k=%d needs more than 64 KiB of LDS", B, layer->hidden,
                layer->n_experts, layer->top_k);
  if (!aligned16(h) || !aligned16(ws) || (z_out && !aligned16(z_out)) || (y_out && !aligned16(y_out)))
    return fail(MOE_ERR_ALIGN, "h, ws, z_out and y_out must be 16-byte aligned");
  {
    // z_out / y_out must not overlap h (the one-kernel path reads h while they are written) or each other
    const size_t n = (size_t)B * layer->hidden * 2;
    auto overlap = [n](const void* a, const void* b) {
      if (!a || !b) return false;
      const uint8_t* p = static_cast<const uint8_t*>(a);
      const uint8_t* q = static_cast<const uint8_t*>(b);
      return p < q + n && q < p + n;
    };
    if (overlap(z_out, h) || overlap(y_out, h) || overlap(z_out, y_out))
      return fail(MOE_ERR_SHAPE, "z_out and y_out must not overlap h or each other");
  }
  const size_t need = carve_decode(layer, B, nullptr, nullptr);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  moe::DecodeWs w;
  carve_decode(layer, B, static_cast<uint8_t*>(ws), &w);
  return hip_status(moe::launch_stack_decode(to_dev(layer), static_cast<uint16_t*>(h), B, eps,
                                             static_cast<uint16_t*>(z_out), static_cast<uint16_t*>(y_out), topk_idx,
                                             topk_gate, w, stream),
                    "moe_stack_decode_layer launch");
}

moe_status moe_forward_prefill(const moe_layer* layer, const void* x, int32_t T, void* y, int32_t* topk_idx,
                               float* topk_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws) return fail(MOE_ERR_NULL, "x, y and ws are required");
  if (T < 1 || T > PREFILL_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "T=%d not in [1, %d]", T, PREFILL_MAX_TOKENS);
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return fail(MOE_ERR_ALIGN, "x, y and ws must be 16-byte aligned");
  const size_t need = carve_prefill(layer, T, nullptr, nullptr);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  moe::PrefillWs w;
  carve_prefill(layer, T, static_cast<uint8_t*>(ws), &w);
  return hip_status(moe::launch_prefill(to_dev(layer), static_cast<const uint16_t*>(x), T, static_cast<uint16_t*>(y),
                                        topk_idx, topk_gate, w, stream),
                    "moe_forward_prefill launch");
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return fail(MOE_ERR_NULL, "ws is required");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "ws must be 16-byte aligned");
  if (ws_bytes < DECODE_SYNC_BYTES) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, DECODE_SYNC_BYTES);
  // the whole workspace: counts and epoch, and the tagged hand-off words (a
  // word left by an earlier owner of the memory must not carry a current tag)
  return hip_status(moe::launch_fill(ws, ws_bytes & ~(size_t)3, stream), "moe_workspace_init launch");
}

moe_status moe_workspace_check(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return fail(MOE_ERR_NULL, "ws is required");
  if (ws_bytes < DECODE_SYNC_BYTES) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, DECODE_SYNC_BYTES);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "moe_workspace_check sync");
  uint32_t flags = 0;
  e = hipMemcpy(&flags, ws, sizeof flags, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "moe_workspace_check read");
  if (flags == 0) return ok();
  const uint32_t zero = 0;
  e = hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e, "moe_workspace_check clear");
  return fail(MOE_ERR_DEVICE, "a device-side wait ran out (flags 0x%x); results since the last check are invalid", flags);
}

moe_status moe_rmsnorm(const void* h, void* z, int32_t T, int32_t H, float eps, hipStream_t stream) {
  if (!h || !z) return fail(MOE_ERR_NULL, "h and z are required");
  if (T < 1 || H < 8 || H % 8 || H > 65536) return fail(MOE_ERR_SHAPE, "T=%d H=%d (H multiple of 8)", T, H);
  if (!aligned16(h) || !aligned16(z)) return fail(MOE_ERR_ALIGN, "h and z must be 16-byte aligned");
  if (!(eps >= 0.0f)) return fail(MOE_ERR_SHAPE, "eps must be >= 0");
  return hip_status(moe::launch_rmsnorm(static_cast<const uint16_t*>(h), static_cast<uint16_t*>(z), T, H, eps, stream),
                    "moe_rmsnorm launch");
}

moe_status moe_residual_add(void* h, const void* y, int32_t T, int32_t H, hipStream_t stream) {
  if (!h || !y) return fail(MOE_ERR_NULL, "h and y are required");
  if (T < 1 || H < 8 || H % 8) return fail(MOE_ERR_SHAPE, "T=%d H=%d (H multiple of 8)", T, H);
  if (!aligned16(h) || !aligned16(y)) return fail(MOE_ERR_ALIGN, "h and y must be 16-byte aligned");
  return hip_status(moe::launch_residual(static_cast<uint16_t*>(h), static_cast<const uint16_t*>(y), T, H, stream),
                    "moe_residual_add launch");
}

// ---------------------------------------------------------------------------
// Host packing
// ---------------------------------------------------------------------------
static moe_status pack_rows(int32_t wt, int32_t rows, int32_t K, const void* const* rsrc,
                            const uint16_t* const* rscale, uint8_t* out, uint16_t* out_scales) {
  const int cb = chunk_bytes(wt), kc = chunk_elems(wt);
  const int nc = K / kc;
  for (int r = 0; r < rows; r++) {
    if (wt == MOE_W_Q4 || wt == MOE_W_Q3) {
      const int8_t* q = static_cast<const int8_t*>(rsrc[r]);
      const int lo = (wt == MOE_W_Q4) ? -8 : -4, hi = (wt == MOE_W_Q4) ? 7 : 3;
      for (int c = 0; c < nc; c++) {
        uint32_t u[32];
        for (int i = 0; i < 32; i++) {
          const int v = q[32 * c + i];
          if (v < lo || v > hi) return fail(MOE_ERR_VALUE, "code %d at row %d col %d outside [%d, %d]", v, r, 32 * c + i, lo, hi);
          u[i] = (uint32_t)(v - lo);
        }
        uint8_t* dst = out + ((size_t)c * rows + r) * cb;
        if (wt == MOE_W_Q4) {
          for (int j = 0; j < 4; j++) {
            uint32_t w = 0;
            for (int s = 0; s < 4; s++) {
              w |= u[8 * j + 2 * s] << (4 * s);
              w |= u[8 * j + 2 * s + 1] << (16 + 4 * s);
            }
            memcpy(dst + 4 * j, &w, 4);
          }
        } else {
          // pairs 0..14: word i / 5, fields at 3 (i % 5) and 16 + 3 (i % 5);
          // pair 15: bit b of elements 30 and 31 at bits 15 and 31 of word b
          uint32_t w[3] = {0, 0, 0};
          for (int i = 0; i < 15; i++) {
            w[i / 5] |= u[2 * i] << (3 * (i % 5));
            w[i / 5] |= u[2 * i + 1] << (16 + 3 * (i % 5));
          }
          for (int b = 0; b < 3; b++) {
            w[b] |= ((u[30] >> b) & 1u) << 15;
            w[b] |= ((u[31] >> b) & 1u) << 31;
          }
          memcpy(dst, w, 12);
        }
        if (out_scales) out_scales[(size_t)c * rows + r] = rscale[r][c];
      }
    } else {
      const int es = (wt == MOE_W_F32) ? 4 : 2;
      const uint8_t* src = static_cast<const uint8_t*>(rsrc[r]);
      for (int c = 0; c < nc; c++) memcpy(out + ((size_t)c * rows + r) * cb, src + (size_t)c * kc * es, cb);
    }
  }
  return ok();
}

moe_status moe_pack_matrix(int32_t wt, int32_t rows, int32_t K, const void* src, const uint16_t* src_scales, void* out,
                           uint16_t* out_scales) {
  if (!is_expert_wt(wt)) return fail(MOE_ERR_DTYPE, "wt=%d unsupported", wt);
  if (rows < 1 || K < 32 || K % 32) return fail(MOE_ERR_SHAPE, "rows=%d K=%d (K multiple of 32)", rows, K);
  if (!src || !out) return fail(MOE_ERR_NULL, "src and out are required");
  if (is_quant(wt) && (!src_scales || !out_scales)) return fail(MOE_ERR_NULL, "scales are required for Q4/Q3");
  const int es = (wt == MOE_W_F32) ? 4 : (wt == MOE_W_BF16) ? 2 : 1;
  std::vector<const void*> rp(rows);
  std::vector<const uint16_t*> sp(rows, nullptr);
  for (int r = 0; r < rows; r++) {
    rp[r] = static_cast<const uint8_t*>(src) + (size_t)r * K * es;
    if (src_scales) sp[r] = src_scales + (size_t)r * (K / 32);
  }
  return pack_rows(wt, rows, K, rp.data(), sp.data(), static_cast<uint8_t*>(out), out_scales);
}

moe_status moe_pack_gate_up(int32_t wt, int32_t I, int32_t H, const void* gate, const uint16_t* gate_scales,
                            const void* up, const uint16_t* up_scales, void* out, uint16_t* out_scales) {
  if (!is_expert_wt(wt)) return fail(MOE_ERR_DTYPE, "wt=%d unsupported", wt);
  if (I < 16 || I % 16 || H < 32 || H % 32) return fail(MOE_ERR_SHAPE, "I=%d (multiple of 16) H=%d (multiple of 32)", I, H);
  if (!gate || !up || !out) return fail(MOE_ERR_NULL, "gate, up and out are required");
  if (is_quant(wt) && (!gate_scales || !up_scales || !out_scales))
    return fail(MOE_ERR_NULL, "scales are required for Q4/Q3");
  const int es = (wt == MOE_W_F32) ? 4 : (wt == MOE_W_BF16) ? 2 : 1;
  const int R = 2 * I;
  std::vector<const void*> rp(R);
  std::vector<const uint16_t*> sp(R, nullptr);
  for (int r = 0; r < R; r++) {
    const int q = r / 32, w = r % 32;
    const bool is_up = w >= 16;
    const int src_row = 16 * q + (w & 15);
    rp[r] = static_cast<const uint8_t*>(is_up ? up : gate) + (size_t)src_row * H * es;
    if (is_quant(wt)) sp[r] = (is_up ? up_scales : gate_scales) + (size_t)src_row * (H / 32);
  }
  return pack_rows(wt, R, H, rp.data(), sp.data(), static_cast<uint8_t*>(out), out_scales);
}

// ---------------------------------------------------------------------------
// Diagnostics
// ---------------------------------------------------------------------------
const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "bad shape";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_DTYPE: return "unsupported weight type";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_VALUE: return "value out of range";
    case MOE_ERR_DEVICE: return "device-side wait ran out";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_debug_set_wait_limit(uint64_t ticks) {
  moe::decode1_set_wait_ticks(ticks);
  return ok();
}

int32_t moe_kernel_class_count(void) { return moe::KC_COUNT; }

const char* moe_kernel_class_name(int32_t id) {
  if (id < 0 || id >= moe::KC_COUNT) return "";
  return kKernelNames[id];
}

moe_status moe_timer_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timer_on = on != 0;
  return ok();
}

moe_status moe_timer_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  drain_locked();
  for (int i = 0; i < moe::KC_COUNT; i++) {
    g_launches[i] = 0;
    g_ms[i] = 0.0;
  }
  return ok();
}

moe_status moe_timer_read(int32_t id, int64_t* launches, double* total_ms) {
  if (id < 0 || id >= moe::KC_COUNT) return fail(MOE_ERR_SHAPE, "kernel class %d out of range", id);
  std::lock_guard<std::mutex> lk(g_tmu);
  drain_locked();
  if (launches) *launches = g_launches[id];
  if (total_ms) *total_ms = g_ms[id];
  return ok();
}

}  // extern "C"
