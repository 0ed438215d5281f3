/*
 * moe_oracle.h -- plain CPU reference for the sparse MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle exists so that tests, the smoke
 * check and the CPU-baseline leg of the benchmark can check the GPU library
 * against an independent, obviously correct computation.  It shares no code,
 * header, table or helper with the GPU library, and the product path never
 * calls it.
 *
 * What it computes (the definition, written out, per token and per selected
 * expert, in fp32 after explicit dequantisation):
 *
 *   out[h] = sum_j score[j] * down_j( silu(gate_j(x)) * up_j(x) )[h]
 *
 * as stated in "perf(moe): fused MoE expert decode kernel, correctness-
 * validated" (lablup/mlxcel #275), section "What it does"; the fp32 reference
 * on dequantised weights follows "SwitchGLU: grouped-expert Metal kernels for
 * small batches of 4-bit experts" (ml-explore/mlx-lm #2044), section
 * "Accuracy"; the dispatch arrays follow DS4Server issue #112, section
 * "Current upstream route" (sort_rows: order, inv_order, row_map) and
 * "Kernel contract" (per-expert row/tile prefix tables).
 *
 * Readings the pages leave open (router accumulation order, tie-break, slot
 * order, q4 packing, shared experts) are fixed in the comments of
 * moe_oracle.c next to the code that implements them.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t d_model;           /* hidden size d */
  int32_t d_ff;              /* per-expert intermediate size */
  int32_t n_experts;         /* routed experts E */
  int32_t top_k;             /* experts selected per token */
  int32_t n_shared;          /* always-on shared experts, weight 1.0 */
  int32_t act_bf16;          /* 0: x, W_router, dense weights are fp32; 1: bf16 */
  int32_t w_q4;              /* 0: dense weights in the activation dtype; 1: affine quantised */
  int32_t group_size;        /* quantisation group length along the reduction dim (32, 64, 128) */
  int32_t gate_up_fused;     /* 1: one [2*d_ff][d] matrix per expert, rows = [gate | up] */
  int32_t glu_round; /* 1: per-op rounding to the activation dtype (bf16 or fp16) in the gated epilogue */
  int32_t renormalize;       /* 1: selected weights renormalised to sum to one */
  int32_t w_bits;            /* affine code width: 4 or 8 */
  int32_t activation;        /* 0: SwiGLU (silu(g) * u); 1: GeGLU with tanh-GELU (gelu(g) * u) */
  int32_t act_f16;           /* 1 (with act_bf16 = 0): x, W_router, dense weights and the
                                affine scales/biases are fp16 */
} oracle_desc;

/* One projection for all experts (routed first, then shared).  Dense:
 * w = [n_all][N][K] in the activation dtype.  Affine b-bit (b = 4 or 8):
 * w = uint32 [n_all][N][K*b/32] (32/b codes per word, code m at bits
 * [b*m, b*m+b) holds column (32/b)*word+m), scales/biases = bits of the
 * 16-bit activation dtype (bf16, or fp16 with act_f16) [n_all][K/group][N]
 * (group-major). */
typedef struct {
  const void *w;
  const uint16_t *scales;
  const uint16_t *biases;
} oracle_proj;

typedef struct {
  oracle_proj gate, up, gate_up, down;
} oracle_experts;

/* Conversions (exposed so tests can pin them against a library cast). */
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
float oracle_f16_to_f32(uint16_t h);
/* fp32 -> binary16 bits, round to nearest even (subnormals, overflow to inf). */
uint16_t oracle_f32_to_f16(float f);

/* Router logits [T][E] in the canonical fp32 order. */
void oracle_router_logits(const oracle_desc *d, int32_t T, const void *x,
                          const void *w_router, const float *router_bias,
                          float *logits);

/* Top-k indices [T][k] and weights [T][k]. */
void oracle_route(const oracle_desc *d, int32_t T, const void *x,
                  const void *w_router, const float *router_bias,
                  int32_t *topk_idx, float *topk_w);

/* Stable grouping of the T*k routed slots by expert. */
void oracle_dispatch(int32_t T, int32_t top_k, int32_t n_experts,
                     const int32_t *topk_idx, int32_t tile_rows,
                     int32_t *order, int32_t *inv_order, int32_t *row_map,
                     int32_t *expert_off, int32_t *tile_off);

/* Dequantised row n of expert e's projection p (K = reduction length). */
void oracle_dequant_row(const oracle_desc *d, const oracle_proj *p, int32_t e,
                        int32_t n, int32_t N, int32_t K, float *out);

/* One expert (index e < E + n_shared) applied to one token row x_row (given
 * in the activation dtype): out[d_model] = down(swiglu(gate x, up x)).
 * h_out (nullable) receives the d_ff SwiGLU values. */
void oracle_expert_apply(const oracle_desc *d, const oracle_experts *w,
                         int32_t e, const void *x_row, float *h_out,
                         float *out);

/* Full layer forward for the tokens listed in `tokens` (n_tok of them, each
 * in [0, T)); y[n_tok][d_model] fp32, topk_idx/topk_w [n_tok][k] (nullable).
 * n_threads <= 0 uses the OpenMP default. */
void oracle_forward_tokens(const oracle_desc *d, int32_t T, const void *x,
                           const void *w_router, const float *router_bias,
                           const oracle_experts *w, int32_t n_tok,
                           const int32_t *tokens, float *y, int32_t *topk_idx,
                           float *topk_w, int32_t n_threads);

/* Backward of the layer with respect to x for the tokens listed in
 * `tokens`: dy[n_tok][d_model] (fp32, row r belongs to tokens[r]) gives
 * dx[n_tok][d_model] = dy . dy/dx at x[tokens[r]], weights fixed, routing
 * fixed at the forward's choice, per-op rounding left out. */
void oracle_backward_tokens(const oracle_desc *d, int32_t T, const void *x,
                            const void *w_router, const float *router_bias,
                            const oracle_experts *w, int32_t n_tok,
                            const int32_t *tokens, const float *dy, float *dx,
                            int32_t n_threads);

/* Threads the last oracle_forward_tokens call ran with. */
int32_t oracle_last_threads(void);

#ifdef __cplusplus
}
#endif
#endif
