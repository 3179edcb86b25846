/*
 * moe_oracle.h - plain CPU oracle of one decode step of a fine-grained MoE
 * layer (and of a stack of such layers).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline of the benchmark may call it. The product path (libmoedecode)
 * never includes, links or calls anything here, and this code shares nothing
 * with it.
 *
 * What it computes, and where that comes from:
 *   - The per-token layer is RMSNorm, a router over all experts, softmax with
 *     top-k selection and renormalisation, a SwiGLU FFN per selected expert,
 *     a shared expert and the residual add. Decode is normalisation, matmul,
 *     activation and routing ops run one after another ("Kimi K3 ... 1.68x",
 *     openai-hub.com, section on why decode suits a megakernel); the layer has
 *     router scores and a shared expert (smzdm.com post, section "what
 *     changed: 23 -> 13 kernels per layer", the MoE de-duplication item);
 *     each token uses 16 of 896 experts (aiposthub.com article, section on
 *     what the K3 decode path changed). The pages print no formula for the
 *     layer; the formula y = x + shared(xhat) + sum_e w_e expert_e(xhat) and
 *     every rounding point below are the readings listed in the design doc.
 *   - Dot products are accumulated in double and rounded once to float where
 *     the layer holds fp32 values; activations that the layer stores in the
 *     activation dtype (the normalised input fed to the FFNs, the SiLU*up
 *     product, the output) are rounded to that dtype (bf16 round to nearest
 *     even, or kept as fp32).
 *
 * All pointers are host pointers. Functions return 0 on success and a
 * negative number on a bad argument (see orc_error_string).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2 };

typedef struct {
  int32_t hidden;        /* H */
  int32_t num_experts;   /* E */
  int32_t top_k;         /* k */
  int32_t expert_inter;  /* I  */
  int32_t shared_inter;  /* Is (0 = no shared expert) */
  float rms_eps;
  int32_t act;           /* dtype of x, y and gamma: ORC_F32 or ORC_BF16 */
  int32_t router;        /* dtype of the router weight: ORC_F32 or ORC_BF16 */
  int32_t expert;        /* dtype of the expert weights: ORC_BF16, ORC_F32 or ORC_FP8_E4M3 */
  int32_t shared;        /* dtype of the shared-expert weights: ORC_F32 or ORC_BF16 */
  int32_t scale_group;   /* rows per bf16 scale for fp8 weights (128) */
} orc_desc;

typedef struct {
  const void *rms_gamma;                        /* [H], act dtype */
  const void *router_w;                         /* [E][H], router dtype */
  const float *router_bias;                     /* [E] or NULL */
  const void *const *expert_gate_up;            /* E pointers to [2I][H] (gate rows, then up rows); NULL = absent */
  const void *const *expert_down;               /* E pointers to [H][I] */
  const uint16_t *const *expert_gate_up_scale;  /* fp8: E pointers to bf16 [2I/G] */
  const uint16_t *const *expert_down_scale;     /* fp8: E pointers to bf16 [H/G] */
  const void *shared_gate_up;                   /* [2Is][H], shared dtype */
  const void *shared_down;                      /* [H][Is] */
} orc_weights;

/* number codecs, written out from the formats' definitions */
double orc_bf16_value(uint16_t bits);
uint16_t orc_bf16_round(double v);       /* v is first rounded to float, then to bf16 (RNE) */
double orc_e4m3_value(uint8_t code);     /* OCP E4M3FN */

/* steps of one token */
int orc_rmsnorm(const orc_desc *d, const void *x_t, const void *gamma, float *xhat, float *xact);
int orc_router_logits(const orc_desc *d, const orc_weights *w, const float *xhat, float *logits);
int orc_route(const orc_desc *d, const float *logits, int32_t *idx, float *wts);
/* weights of a given selection idx [k] (distinct, in range): restricted, renormalised softmax */
int orc_route_weights(const orc_desc *d, const float *logits, const int32_t *idx, float *wts);
int orc_ffn(const orc_desc *d, int32_t dtype, int32_t inter, const void *gate_up, const void *down,
            const uint16_t *gate_up_scale, const uint16_t *down_scale, const float *xact,
            float *h_out, float *d_out);

/* one token through one layer; logits may be NULL */
int orc_layer_token(const orc_desc *d, const orc_weights *w, const void *x_t, void *y_t,
                    int32_t *idx, float *wts, float *logits);
/* one token through one layer with the caller's selection idx [k] (rank order) in place of
 * the top-k; wts receives that selection's weights; logits may be NULL */
int orc_layer_token_given(const orc_desc *d, const orc_weights *w, const void *x_t, const int32_t *idx,
                          void *y_t, float *wts, float *logits);
/* B tokens: x, y [B][H] act dtype; idx, wts [B][k]; logits [B][E] or NULL */
int orc_layer(const orc_desc *d, const orc_weights *w, const void *x, int32_t B, void *y,
              int32_t *idx, float *wts, float *logits);
/* L layers, each with its own weights: y = layer_{L-1}(...layer_0(x)); idx, wts [L][B][k];
 * logits [L][B][E] or NULL */
int orc_stack(const orc_desc *d, const orc_weights *layers, int32_t L, const void *x, int32_t B,
              void *y, int32_t *idx, float *wts, float *logits);

const char *orc_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif
