/*
 * moe.h - C ABI of the quantized routed-expert MoE layer for AMD MI355X (gfx950).
 *
 * One layer of a sparse Mixture-of-Experts model: a router picks k of E
 * routed experts per token (the pages' model uses 10 of 512, plus one shared
 * expert that always runs: Strata write-up, "The 30-Second Overview" table;
 * explainer video, transcript at 2:01). Each selected expert is a SwiGLU FFN
 * whose weights are block-quantised (the pages run 2-3.5 bit experts: write-up
 * section 1 "Low-Bit Quantization"); the outputs of a token's experts are
 * summed into one result (video, transcript at 3:36). The router, gate and
 * FFN formulas are not on the pages; this library computes:
 *
 *   l_e  = sum_h W_r[e,h] x[h] + b_e                 (fp64 accumulation)
 *   S    = k largest l_e, ordered by (l_e desc, e asc)
 *   g_i  = softmax over all E, renormalised over S   (= softmax of l_S)
 *   y    = sum_i g_i * D_{S_i}( SiLU(G_{S_i} x) * (U_{S_i} x) )
 *          + D_s( SiLU(G_s x) * (U_s x) )            (shared expert, weight 1)
 *
 * with w = fp16_scale * signed_code for quantised weights (blocks of 32
 * consecutive elements along the input dimension).
 *
 * CONVENTIONS
 *  - Every pointer passed to a compute entry point is DEVICE memory owned by
 *    the caller. The library never allocates device memory, never holds state
 *    between calls (except the counters of the optional kernel timer) and
 *    never synchronises the stream: calls enqueue work on `stream` and
 *    return. Calls are graph-capturable (no memset nodes, no host syncs).
 *  - Arguments are validated on the host before anything is enqueued. A
 *    failing call returns a non-zero moe_status and enqueues nothing. A HIP
 *    launch failure returns MOE_ERR_HIP; moe_last_error() describes it.
 *  - Device pointers must be 16-byte aligned.
 *  - Activations are bf16 (uint16 bit patterns) in and out, row-major [T][H].
 *  - Two calls that share one workspace must be ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of range or not a multiple it must be */
  MOE_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
  MOE_ERR_DTYPE = 4,     /* unsupported weight type or combination */
  MOE_ERR_WORKSPACE = 5, /* workspace too small */
  MOE_ERR_HIP = 6,       /* a HIP runtime call failed */
  MOE_ERR_VALUE = 7,     /* host packing: a code is outside its type's range */
  MOE_ERR_DEVICE = 8     /* a device-side wait ran out (reported by moe_workspace_check) */
} moe_status;

/* Weight storage types. */
typedef enum {
  MOE_W_F32 = 0,   /* fp32 values */
  MOE_W_BF16 = 1,  /* bf16 values */
  MOE_W_Q4 = 2,    /* signed 4-bit codes in [-8,7], one fp16 scale per 32-element block */
  MOE_W_Q3 = 3,    /* signed 3-bit codes in [-4,3], one fp16 scale per 32-element block */
  MOE_W_NONE = -1  /* no shared expert */
} moe_wtype;

/*
 * PACKED WEIGHT LAYOUT (the library's own; produce it with moe_pack_matrix)
 *
 * A weight matrix W[R][K] (R output rows, K input elements, K % 32 == 0) is
 * stored "chunk-major": the K axis is cut into chunks, and chunk c of every
 * row is stored before chunk c+1 of any row:
 *
 *     value bytes : [K / kc][R][cb]      scales : [K / 32][R]  (fp16)
 *
 *   F32 : kc = 4 elements,  cb = 16 bytes (4 x fp32)
 *   BF16: kc = 8 elements,  cb = 16 bytes (8 x bf16)
 *   Q4  : kc = 32 elements, cb = 16 bytes = four little-endian 32-bit words
 *         w0..w3; word j holds elements 8j..8j+7 as unsigned (code + 8):
 *         element 8j+2s   at bits [4s, 4s+4),
 *         element 8j+2s+1 at bits [16+4s, 16+4s+4),   s = 0..3
 *   Q3  : kc = 32 elements, cb = 12 bytes = three little-endian 32-bit
 *         words w0, w1, w2 holding the unsigned (code + 4) in [0,7]:
 *         for i = 0..14, with m = i / 5 and s = i % 5, element 2i at
 *         bits [3s, 3s+3) of word m and element 2i+1 at bits
 *         [16+3s, 16+3s+3) of word m;
 *         elements 30 and 31: bit b (b = 0..2) of element 30 at bit 15 of
 *         word b, bit b of element 31 at bit 31 of word b.
 *   F32 and BF16 matrices have no scales.
 *
 * An expert's gate and up projections (each [I][H]) are fused into one
 * matrix GU[2I][H] whose rows come in groups of 32: rows 32q..32q+15 are
 * gate rows 16q..16q+15 and rows 32q+16..32q+31 are up rows 16q..16q+15
 * (I % 16 == 0). The down projection is D[H][I].
 *
 * Routed experts are stored back to back: expert e's fused gate/up values
 * start at byte e * moe_matrix_bytes(wt, 2I, H) of gate_up, its scales at
 * element e * moe_matrix_scales(wt, 2I, H) of gate_up_scales; likewise for
 * down with (H, I).
 */
typedef struct {
  int32_t hidden;          /* H: multiple of 32, 32..8192 */
  int32_t inter;           /* I: multiple of 32, 32..4096 */
  int32_t n_experts;       /* E: 1..1024 */
  int32_t top_k;           /* k: 1..min(16, E) */
  const float *router_w;   /* [E][H] fp32 row-major */
  const float *router_bias;/* [E] fp32, or NULL for no bias */
  int32_t expert_wtype;    /* moe_wtype of the routed experts: F32, BF16, Q4 or Q3 */
  const void *gate_up;     /* packed [E] x GU[2I][H] */
  const uint16_t *gate_up_scales; /* fp16, NULL for F32/BF16 */
  const void *down;        /* packed [E] x D[H][I] */
  const uint16_t *down_scales;    /* fp16, NULL for F32/BF16 */
  int32_t shared_wtype;    /* F32, BF16 or MOE_W_NONE */
  const void *shared_gate_up;     /* packed GU[2I][H] of the shared expert */
  const void *shared_down;        /* packed D[H][I] of the shared expert */
} moe_layer;

/* ------------------------------------------------------------------------ */
/* Sizes and workspace                                                      */
/* ------------------------------------------------------------------------ */

/* Sizes of the library's own packed layout above (the pages give no storage
 * format; they only put the experts at 2-3.5 bits per weight: Strata
 * write-up, section 1 "Low-Bit Quantization"). */
/* Bytes of packed values of one R x K matrix of type wt (0 on bad input). */
size_t moe_matrix_bytes(int32_t wt, int32_t rows, int32_t K);
/* Number of fp16 scales of one R x K matrix (0 for F32/BF16). */
size_t moe_matrix_scales(int32_t wt, int32_t rows, int32_t K);

/* Workspace bytes needed by moe_route / moe_forward_decode (mode 0, up to
 * max_tokens <= MOE_DECODE_MAX_TOKENS tokens per call) or
 * moe_forward_prefill (mode 1, up to max_tokens tokens per call). Returns 0
 * when the layer or sizes are invalid. */
size_t moe_workspace_bytes(const moe_layer *layer, int32_t max_tokens, int32_t mode);
#define MOE_DECODE_MAX_TOKENS 8

/* Workspace contract (the library's own). A decode workspace must be all
 * zero before its first decode call: moe_workspace_init zero-fills all
 * ws_bytes (as would any zero fill). Its first 4096 bytes hold the counts and the call epoch of the
 * one-kernel decode paths; the rest holds the words through which their
 * workgroups hand data to each other: every flag, and every value not
 * guarded by a flag, carries the call's tag (a word counts only when it
 * carries the current call's tag, so memory left by an earlier owner must
 * not be reused uninitialised). Every call leaves the counts zero and advances the epoch,
 * so the workspace can be reused call after call and inside captured HIP
 * graphs. Calls that share one workspace must be ordered (one stream);
 * concurrent calls on one workspace race. Prefill workspaces need no
 * initialisation. */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Synchronises `stream`, then reports whether a device-side wait of a
 * decode call on this workspace ran out of time since the last check
 * (MOE_ERR_DEVICE: results of those calls are invalid) and clears the
 * report. The one-kernel decode paths (batch 1 and 2..8) need all of their
 * workgroups resident at once (some wait for others); the library checks that the
 * grid fits the device, but other work on the GPU (other streams, other
 * processes) can hold compute units long enough for a wait to reach its
 * bound (moe_debug_set_wait_limit; about 0.34 s by default). The bound
 * exists so that the kernel always ends; this call is how a caller learns
 * that it ended early. Callers that share the GPU should check after a run
 * of calls. (No passage of the pages: the check is the library's own.) */
moe_status moe_workspace_check(void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Compute entry points                                                     */
/* ------------------------------------------------------------------------ */

/* Routing only (router GEMV/GEMM, softmax, ordered top-k, renormalised
 * gates) for T >= 1 tokens x[T][H] (bf16). Each layer's router picks k of
 * the E routed experts for every token, 10 of 512 in the pages' model
 * (explainer video, transcript at 1:50-2:01; Strata write-up, "The
 * 30-Second Overview" table); the routers stay resident on the GPU (video
 * at 2:28-2:38). The router formula, the gate normalisation and the tie
 * rule are not on the pages: the library's reading is the one in the
 * preamble above.
 *   topk_idx   [T][k] int32   experts in (logit desc, index asc) order
 *   topk_gate  [T][k] fp32    renormalised gates, same order
 *   expert_counts [E] int32 or NULL: number of tokens routed to each expert
 * Workspace: moe_workspace_bytes(layer, T, 1). */
moe_status moe_route(const moe_layer *layer, const void *x, int32_t T,
                     int32_t *topk_idx, float *topk_gate, int32_t *expert_counts,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Decode: B in 1..MOE_DECODE_MAX_TOKENS tokens x[B][H] -> y[B][H] (bf16).
 * The token's k selected experts and the always-on shared expert, their
 * outputs summed into the token's one result (explainer video, transcript
 * at 2:01 and 3:36); a decode step is paced by the expert bytes it has to
 * move (Strata write-up, "How Strata Makes It Run" section 2 "Expert Cache
 * and CPU/GPU Split"). B > 1 serves the short batches of speculative
 * verification (write-up section 4 "MTP Speculative Decoding"; video at
 * 5:09), whose drafts are a handful of tokens: B is capped at 8, not 16.
 * (B * H * 2 bytes of activations are staged in LDS: B * H must not exceed
 * 8 * 2048; larger requests return MOE_ERR_SHAPE.)
 * Batch-1 decode is bound by the bytes of the selected experts' weights: a
 * fused dequantise-GEMV streams each selected expert once per call (experts
 * chosen by several tokens of the batch are read once). B = 1 runs as one
 * kernel (router, top-k, gate/up, SwiGLU, down and combine) when
 * E <= 512, H <= 2048 and I <= 1024; otherwise, and for B > 1, as four
 * kernels (router and shared expert, routing of the batch, routed experts,
 * sum of the partial products). topk_idx/topk_gate ([B][k]) are optional outputs (NULL to
 * skip). Workspace: moe_workspace_bytes(layer, B, 0), initialised once as
 * described above. */
moe_status moe_forward_decode(const moe_layer *layer, const void *x, int32_t B, void *y,
                              int32_t *topk_idx, float *topk_gate,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device array of the library instead of the caller's. The array,
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, exists on every device the
 * library runs on until the process ends; this call allocates nothing.
 * Arguments and outputs as moe_forward_decode; a layer and B whose
 * workspace (moe_workspace_bytes(layer, B, 0)) exceeds the array return
 * MOE_ERR_WORKSPACE and enqueue nothing.
 * The first call on a device sets the array up: it looks up the array's
 * device address, zeroes the array on `stream` and waits for that, so it
 * must not be under graph capture (MOE_ERR_SHAPE if it is); later calls are
 * stream-ordered and capturable. All calls on one GPU share its array, so
 * calls that may overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller. The device-side wait report of these
 * calls stays in the array (moe_workspace_check needs a caller workspace). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_decode_noalloc(const moe_layer *layer, const void *x, int32_t B, void *y,
                                      int32_t *topk_idx, float *topk_gate, hipStream_t stream);

/* Prefill: T >= 1 tokens x[T][H] -> y[T][H] (bf16). Prompts are taken in
 * large pieces, up to 8,192 tokens (Strata README, "How does it work"), and
 * the prompt's experts run on matrix-core kernels (4090 report, "Fused
 * prefill kernels"); the arithmetic is that of moe_forward_decode for every
 * token. Tokens are grouped by
 * expert (histogram, exclusive scan, stable permutation) and each expert's
 * tokens go through an MFMA grouped GEMM with the expert's weights
 * dequantised to bf16 in LDS; a gather combine adds the gated expert
 * outputs in slot order and the shared expert. topk_idx/topk_gate ([T][k])
 * are optional outputs. Workspace: moe_workspace_bytes(layer, T, 1). */
moe_status moe_forward_prefill(const moe_layer *layer, const void *x, int32_t T, void *y,
                               int32_t *topk_idx, float *topk_gate,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* Between stacked layers (pre-norm residual stream). The pages' model has
 * 48 such MoE layers (Strata write-up, section 2; explainer video at 1:37)
 * but give no layer formula: the plain pre-norm residual form is the
 * library's reading.
 *   moe_rmsnorm:      z = h / sqrt(mean(h^2) + eps), unit gain, fp32 math
 *   moe_residual_add: h = bf16(h + y)
 * h, z, y: bf16 [T][H]. */
moe_status moe_rmsnorm(const void *h, void *z, int32_t T, int32_t H, float eps, hipStream_t stream);
moe_status moe_residual_add(void *h, const void *y, int32_t T, int32_t H, hipStream_t stream);

/* One decode step of a stacked layer (the pages give no layer formula; the
 * stack's form is the plain pre-norm residual one), in place on the
 * residual stream h (bf16 [B][H], B in 1..MOE_DECODE_MAX_TOKENS): z = RMSNorm(h) as
 * moe_rmsnorm computes it, y = moe_forward_decode(z), h = bf16(h + y) as
 * moe_residual_add computes it. At batch 1, when the one-kernel decode path
 * takes the shape, all three run in that one kernel (every workgroup that
 * reads the token normalises it itself; the reducers add the residual);
 * otherwise as the three calls in turn. z_out, y_out ([B][H] bf16) receive
 * z and y when not NULL and must not overlap h or each other;
 * topk_idx/topk_gate as in moe_forward_decode.
 * Workspace: moe_workspace_bytes(layer, B, 0), as for moe_forward_decode
 * (the two may share one). Errors as moe_forward_decode, and MOE_ERR_SHAPE
 * for eps < 0 or overlapping h, z_out, y_out. */
moe_status moe_stack_decode_layer(const moe_layer *layer, void *h, int32_t B, float eps, void *z_out, void *y_out,
                                  int32_t *topk_idx, float *topk_gate, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Host-side packing (no device work; host pointers)                        */
/* ------------------------------------------------------------------------ */

/* The layout is the library's own (see PACKED WEIGHT LAYOUT; the pages give
 * none). Pack one matrix W[R][K] (row-major source) into the chunk-major layout.
 *   Q4/Q3: src = int8 codes [R][K] (range-checked), src_scales = fp16 [R][K/32]
 *   F32  : src = float [R][K];  BF16: src = uint16 bf16 [R][K]; src_scales NULL
 * out: moe_matrix_bytes(wt,R,K) bytes; out_scales: moe_matrix_scales(wt,R,K)
 * elements (may be NULL for F32/BF16). */
moe_status moe_pack_matrix(int32_t wt, int32_t rows, int32_t K, const void *src,
                           const uint16_t *src_scales, void *out, uint16_t *out_scales);

/* Pack gate [I][H] and up [I][H] into the fused GU[2I][H] described above. */
moe_status moe_pack_gate_up(int32_t wt, int32_t I, int32_t H, const void *gate,
                            const uint16_t *gate_scales, const void *up,
                            const uint16_t *up_scales, void *out, uint16_t *out_scales);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                              */
/* ------------------------------------------------------------------------ */

/* Library diagnostics (no passage of the pages). */
const char *moe_status_string(int32_t status);
/* Description of the last failure on this thread ("" if none). */
const char *moe_last_error(void);

/* Bound of every device-side wait of the one-kernel batch-1 decode, in ticks
 * of the GPU's 100 MHz wall clock, for the calls enqueued after this one
 * (process-wide; 0 restores the default of 2^25 ticks, about 0.34 s). A wait
 * that runs out lets its workgroup finish with invalid results and sets the
 * report read by moe_workspace_check. For tests of that report: a tiny bound
 * makes waits give up while their producers are still running. */
moe_status moe_debug_set_wait_limit(uint64_t ticks);

/* Optional per-kernel timer: when enabled, every kernel the library
 * launches carries a start and a stop HIP event in its own dispatch on its
 * stream (hipExtLaunchKernel), so each interval is that kernel's execution.
 * moe_timer_read waits for the recorded events and returns, for kernel
 * class `id`, the number of launches and their summed duration since the
 * last reset. Not for use under graph capture. */
int32_t moe_kernel_class_count(void);
const char *moe_kernel_class_name(int32_t id);
moe_status moe_timer_enable(int32_t on);
moe_status moe_timer_reset(void);
moe_status moe_timer_read(int32_t id, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
