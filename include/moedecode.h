/*
 * moedecode.h - C ABI of libmoedecode: the decode step of a fine-grained
 * Mixture-of-Experts transformer layer on AMD MI355X (gfx950).
 *
 * The layer (per token t, activation x_t of width H):
 *   xhat    = x_t / sqrt(mean(x_t^2) + eps) * gamma                 (RMSNorm)
 *   l_e     = <Wr[e], xhat> (+ bias_e)        for all E experts      (router)
 *   S       = the k largest l_e, ties to the lower e                 (top-k)
 *   w_e     = softmax(l)_e / sum_{e' in S} softmax(l)_e'             (renormalised)
 *   f_W(v)  = Wd (SiLU(Wg v) * (Wu v))                               (SwiGLU FFN)
 *   y_t     = x_t + f_shared(xhat) + sum_{e in S} w_e f_e(xhat)
 * Decode is a chain of normalisation, matmul, activation and routing ops
 * (openai-hub.com "Kimi K3 ... 1.68x", section on why decode suits a
 * megakernel); the MoE has router scores and a shared expert (smzdm.com
 * post, section "what changed", MoE de-duplication item); Kimi K3 sends each
 * token to 16 of its 896 experts (aiposthub.com article, section on what the
 * K3 decode path changed); the specialised path covers decode batches 1-64
 * and falls back to the stock path elsewhere (smzdm.com post, section on who
 * can use it). The pages give no formula; the one above, its rounding points
 * and tie rule are this library's reading of them.
 *
 * Precision: the router consumes fp32 xhat; the FFNs consume xhat rounded to
 * the activation dtype; SiLU(g)*u is stored in the activation dtype; all dot
 * products accumulate in fp32; y is rounded once to the activation dtype.
 *
 * Conventions for every entry point:
 *   - Pointers inside moe_layer_weights, and x, y, the optional outputs and
 *     the workspace, are DEVICE pointers (hipMalloc or torch memory) on the
 *     current HIP device. desc, weights and the layers array are HOST structs,
 *     read during the call only.
 *   - The caller owns all memory. The library allocates nothing and does not
 *     synchronise: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and pointers must stay valid until it completes.
 *   - Validation is synchronous and happens before any launch. Errors are
 *     returned as moe_status; moe_last_error() gives a thread-local detail.
 *     Device errors of a launch return MOE_ERR_DEVICE.
 *   - Layouts are row-major, [out][in]: the router [E][H]; expert gate/up
 *     [E][2I][H] with the gate rows first, then the up rows; expert down
 *     [E][H][I]; shared gate/up [2Is][H]; shared down [H][Is].
 *   - All device pointers must be 16-byte aligned.
 *   - The workspace must be zero-filled by the caller once, before the first
 *     call that uses it; every call leaves it as it found it (barrier and
 *     work counters back at zero, the small-batch logit buffers cleared), so
 *     it is reusable across calls, batch sizes and layer counts. After a
 *     watchdog stop (MOE_ERR_TIMEOUT from moe_check_workspace, which also
 *     restores that state) no other repair is needed. Calls that share one
 *     workspace must not overlap in time (enqueue them on one stream).
 *   - y may be exactly x (in place); any other overlap between inputs and
 *     outputs is an error.
 *   - Routing outputs list each token's k experts by descending logit, ties
 *     to the lower expert index; weights match that order and sum to 1.
 *   - Co-residency: a fused launch is one 1024-thread workgroup per compute
 *     unit whose grid barriers need every workgroup resident at once. Kernels
 *     of other streams or processes that hold compute units delay it; every
 *     in-kernel wait gives up after the watchdog limit (2 s by default, see
 *     moe_set_watchdog_ticks). A launch in which a wait gave up still
 *     completes, but writes NaN into the rows of y it can no longer trust and
 *     -1 / NaN into every routing output (indices / weights / logits) it
 *     wrote, and moe_check_workspace then returns MOE_ERR_TIMEOUT.
 */
#ifndef MOEDECODE_H
#define MOEDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad size, partial overlap */
  MOE_ERR_UNSUPPORTED = 2,         /* outside the envelope below: the caller falls back */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < moe_workspace_bytes(...) */
  MOE_ERR_DEVICE = 4,              /* a HIP call or kernel launch failed */
  MOE_ERR_TIMEOUT = 5              /* a previous launch hit its grid-barrier watchdog */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Shape and dtypes of one layer (host struct).
 * Envelope (else MOE_ERR_UNSUPPORTED):
 *   hidden % 128 == 0, hidden <= 16384; expert_inter % 128 == 0 and <= 4096;
 *   shared_inter % 128 == 0 (0 = no shared expert) and <= 8192;
 *   1 <= top_k <= 32; top_k <= num_experts <= 1024; batch 1..64; layers 1..8;
 *   dtype sets: {act F32, router F32, expert F32, shared F32},
 *   {act BF16, router F32 or BF16, expert BF16, shared BF16},
 *   {act BF16, router F32 or BF16, expert FP8_E4M3 with scale_group 128, shared BF16}. */
typedef struct {
  int32_t hidden;        /* H */
  int32_t num_experts;   /* E */
  int32_t top_k;         /* k */
  int32_t expert_inter;  /* I: each routed expert's intermediate width */
  int32_t shared_inter;  /* Is: the shared expert's intermediate width (0 = none) */
  float rms_eps;         /* e.g. 1e-6 */
  moe_dtype act;         /* x, y and gamma */
  moe_dtype router;      /* router weight */
  moe_dtype expert;      /* routed expert weights */
  moe_dtype shared;      /* shared expert weights */
  int32_t scale_group;   /* FP8 experts: output rows per bf16 scale (128); else 0 */
} moe_layer_desc;

/* Device pointers of one layer's weights (host struct). */
typedef struct {
  const void *rms_gamma;             /* [H], act dtype */
  const void *router_w;              /* [E][H], router dtype */
  const float *router_bias;          /* [E] fp32 added to the logits, or NULL */
  const void *expert_gate_up;        /* [E][2I][H], expert dtype */
  const void *expert_down;           /* [E][H][I], expert dtype */
  const uint16_t *expert_gate_up_scale; /* FP8: bf16 [E][2I/scale_group]; else NULL */
  const uint16_t *expert_down_scale;    /* FP8: bf16 [E][H/scale_group]; else NULL */
  const void *shared_gate_up;        /* [2Is][H], shared dtype (NULL if Is == 0) */
  const void *shared_down;           /* [H][Is], shared dtype (NULL if Is == 0) */
} moe_layer_weights;

/* Bytes of workspace needed for up to max_tokens tokens and num_layers layers
 * of this shape; 0 if desc is invalid or outside the envelope. */
size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens, int32_t num_layers);

/* Routing only: RMSNorm + router + softmax/top-k/renormalisation for B tokens
 * (the router scores every expert and each token keeps its top 16 of 896 in
 * Kimi K3: smzdm.com post, section "what changed", MoE de-duplication item;
 * aiposthub.com article, section on what the K3 decode path changed).
 *   x        [B][H] act dtype
 *   topk_idx [B][k] int32 out; topk_w [B][k] fp32 out
 *   logits   [B][E] fp32 out (router logits incl. bias), or NULL
 * One kernel launch on `stream`. */
moe_status moe_route(const moe_layer_desc *desc, const moe_layer_weights *weights, const void *x,
                     int32_t B, int32_t *topk_idx, float *topk_w, float *logits, void *ws,
                     size_t ws_bytes, void *stream);

/* The whole layer for B tokens in one persistent kernel launch: the decode
 * step's normalisation, matmul, activation and routing ops fused into one
 * kernel instead of one launch each (openai-hub.com "Kimi K3 ... 1.68x",
 * section on why decode suits a megakernel), the shared expert's work beside
 * the routing (smzdm.com post, section "what changed", MoE de-duplication
 * item), batch 1-64 (smzdm.com post, section on who can use it).
 *   x [B][H] act dtype in; y [B][H] act dtype out (y == x allowed);
 *   topk_idx [B][k] / topk_w [B][k]: the routing used, or NULL. */
moe_status moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *weights,
                            const void *x, void *y, int32_t B, int32_t *topk_idx, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_decode_layer, with the library's own workspace instead of a
 * caller-allocated one, so the call allocates nothing and needs no workspace
 * argument. That workspace is one 16 MiB device array per GPU, held until the
 * process ends, zeroed by a small fill kernel on `stream` at the first call on
 * each device. Shapes whose moe_workspace_bytes(desc, B, 1) exceeds 16 MiB
 * (at the K3 share, H = 7168, E = 896, k = 16, I = 1024, Is = 2048: batches
 * above 26) return MOE_ERR_UNSUPPORTED before any launch. Every call on one
 * GPU shares the array and finds it as the previous call left it: calls that
 * overlap in time on one GPU (other streams or threads) race and give wrong
 * results, so enqueue them on one stream. A watchdog stop shows in the
 * outputs as for moe_decode_layer (NaN rows, -1 / NaN routing); the launch
 * restores the array itself. Other arguments as for moe_decode_layer. */
moe_status moe_decode_layer_static(const moe_layer_desc *desc, const moe_layer_weights *weights,
                                   const void *x, void *y, int32_t B, int32_t *topk_idx, float *topk_w,
                                   void *stream);

/* L layers of the same shape, each with its own weights (layers: host array of
 * L structs), in one persistent launch: y = layer_{L-1}(... layer_0(x)), each
 * layer's bf16 output feeding the next layer's RMSNorm. The layers stay in one
 * launch (openai-hub.com "Kimi K3 ... 1.68x", section on why decode suits a
 * megakernel), separated by one grid barrier. (Warming the next layer's
 * weights during that barrier, the single-GPU form of the pages' next-step
 * prefetch (smzdm.com post, section "what changed", bandwidth-stealing
 * prefetch item), was measured and left out: it slowed every batch.)
 *   topk_idx [L][B][k] / topk_w [L][B][k]: the routing of every layer, or NULL. */
moe_status moe_decode_stack(const moe_layer_desc *desc, const moe_layer_weights *layers, int32_t L,
                            const void *x, void *y, int32_t B, int32_t *topk_idx, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace moe_decode_layer_unfused needs for up to max_tokens
 * tokens of this shape; 0 if desc is invalid or outside the envelope. */
size_t moe_unfused_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens);

/* The same layer as moe_decode_layer, computed by eleven separate kernel
 * launches (RMSNorm, router, top-k, expert grouping, expert gate/up,
 * SiLU*mul, expert down, shared gate/up, shared SiLU*mul, shared down,
 * combine) with every
 * intermediate in device memory: the launch-per-op decode path the pages
 * describe before fusion (openai-hub.com "Kimi K3 ... 1.68x", section on why
 * decode suits a megakernel: many small separately launched norm, matmul,
 * activation and routing kernels; smzdm.com post, section "what changed":
 * 23 kernels and ~130 us per decoder layer before, 13 and ~69 us after). It
 * is the measured baseline of the fused kernel. The grouping kernel sorts
 * the (token, expert) pairs by expert, so each selected expert's rows are
 * read once per group of up to 4 of its tokens.
 *   Arguments as for moe_decode_layer, except the workspace, which is sized
 *   by moe_unfused_workspace_bytes and needs no zero fill (every call writes
 *   it before reading it). topk_idx / topk_w may be NULL (the routing then
 *   stays in the workspace). Same validation and status codes. */
moe_status moe_decode_layer_unfused(const moe_layer_desc *desc, const moe_layer_weights *weights,
                                    const void *x, void *y, int32_t B, int32_t *topk_idx,
                                    float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* Flags of moe_decode_stack_unfused: the side-stream forms the pages give for
 * two of the specialised path's changes (smzdm.com post, section "what
 * changed": the shared expert computed on a second stream beside routing, in
 * the MoE de-dup item; a side kernel that warms the cache with next-step
 * weights while HBM is otherwise idle, in the bandwidth-stealing prefetch
 * item). */
enum {
  MOE_UF_SHARED_SIDE = 1,   /* each layer's shared gate/up, SiLU*mul and down on side_stream,
                               concurrent with its routed path */
  MOE_UF_PREFETCH_SIDE = 2  /* after layer l's RMSNorm, a kernel on side_stream reads layer l+1's
                               router, shared gate/up and shared down weights with cache-allocating
                               loads (nothing for the last layer) */
};

/* Bytes of workspace moe_decode_stack_unfused needs for up to max_tokens
 * tokens and num_layers layers of this shape; 0 if desc is invalid or outside
 * the envelope. At num_layers = 1 it equals moe_unfused_workspace_bytes. */
size_t moe_unfused_stack_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens,
                                         int32_t num_layers);

/* L layers (1..8) of the same shape through the multi-launch path of
 * moe_decode_layer_unfused, each layer's output feeding the next layer's
 * RMSNorm (between layers it lives in the workspace): the same results as
 * moe_decode_stack, with every layer's eleven launches enqueued by this call.
 * flags (0, or MOE_UF_* bits) move work to side_stream; the results do not
 * depend on them (the same kernels on the same data, bit for bit).
 *   layers: host array of L weight structs. topk_idx / topk_w: [L][B][k] or
 *   NULL. ws: moe_unfused_stack_workspace_bytes(desc, B, L) bytes, no zero
 *   fill. stream, side_stream: hipStream_t of the current device;
 *   side_stream may be NULL only when flags is 0. Work on side_stream waits
 *   for `stream` through events and is joined back into `stream` before the
 *   call's last launch, so waiting for `stream` covers all of it. The
 *   library keeps two events per device for this and enqueues one such call
 *   at a time (a mutex). Both streams should have the default priority.
 * Same validation and status codes as moe_decode_layer_unfused; unknown flag
 * bits, or flags without a side stream, are MOE_ERR_INVALID_ARGUMENT. */
moe_status moe_decode_stack_unfused(const moe_layer_desc *desc, const moe_layer_weights *layers,
                                    int32_t L, const void *x, void *y, int32_t B, int32_t *topk_idx,
                                    float *topk_w, void *ws, size_t ws_bytes, void *stream,
                                    void *side_stream, uint32_t flags);

/* Synchronises `stream`, then reads and clears the workspace's error word:
 * MOE_ERR_TIMEOUT if a launch on this workspace stopped at a watchdog (a grid
 * barrier or the small-batch logit wait gave up after the watchdog limit),
 * MOE_OK otherwise.
 * On MOE_ERR_TIMEOUT it also clears the small-batch logit buffers that the
 * stopped launch may have left written. A debugging aid, not for the hot
 * path. */
moe_status moe_check_workspace(void *ws, size_t ws_bytes, void *stream);

/* Limit of every in-kernel wait of later launches (grid barriers, the
 * small-batch logit wait), in ticks of the GPU's 100 MHz realtime counter;
 * a negative value restores the default of 2e8 (2 s). A limit of 0 makes each
 * wait that would block give up at once, which exercises the timeout path
 * (NaN outputs, MOE_ERR_TIMEOUT) without a hang. Process-wide. */
void moe_set_watchdog_ticks(int64_t ticks);

/* Static English name of a status. */
const char *moe_status_string(moe_status status);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEDECODE_H */
