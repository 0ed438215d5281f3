/*
 * moe_mi355x.h -- C ABI of the sparse Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (per token t with row x[t] of length d_model):
 *   1. route:    logits = x[t] . W_router (+ router_bias), softmax, top-k
 *                experts with their weights, renormalised to sum to one;
 *   2. dispatch: the T*k routed (token, slot) rows grouped by expert;
 *   3. experts:  for each routed row, h = silu(x . Wg_e) * (x . Wu_e) and
 *                y_e = h . Wd_e (SwiGLU expert FFN);
 *   4. combine:  y[t] = sum_j w[t][j] * y_{e_j}(x[t]) + sum_s shared_s(x[t]).
 * This is the layer of "perf(moe): fused MoE expert decode kernel" (lablup/
 * mlxcel #275, section "What it does": out = sum_k score_k * down_k(silu(
 * gate_k(x)) * up_k(x))), with the routing kernel contract of the PRD "5.5
 * real sparse MoE kernels (Metal)" (section "Scope - in": routing_logits ->
 * (top_k_indices, top_k_weights) with no host round trip; expert dispatch
 * (tokens, expert_indices) -> grouped tokens; scatter-add combine) and the
 * sorted-row route of DS4Server issue #112 (section "Current upstream
 * route": sort_rows -> order, inv_order, row_map; gate/up SwiGLU reading
 * rows in place through row_map; down on the sorted rows; unsort through
 * inv_order).
 *
 * Conventions shared by every entry point:
 *  - Pointers named as tensors are DEVICE pointers owned by the caller, 16-byte
 *    aligned, to densely packed row-major arrays.  Descriptor/weight-table
 *    structs and `bytes` out-parameters are HOST pointers.
 *  - Each call validates everything on the host first; on any error it returns
 *    a negative moe_status, enqueues nothing and leaves every output untouched.
 *  - On success the work is only ENQUEUED on `stream` (a hipStream_t, NULL =
 *    the default stream).  No call synchronises the host or copies device data
 *    to the host; buffers must stay alive until the stream work completes.
 *  - T == 0 is valid and enqueues nothing.
 *  - The library allocates no device memory: scratch space comes from the
 *    caller's workspace (`ws`, `ws_bytes`, sized by moe_workspace_size).
 *  - Results are deterministic: no floating-point atomics anywhere, so two
 *    identical calls give bitwise identical outputs.
 *  - Calls that share a workspace must not run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = -1,     /* bad descriptor, size, pointer or alignment */
  MOE_E_UNSUPPORTED = -2, /* a valid but unimplemented format (bits, group) */
  MOE_E_WORKSPACE = -3,   /* ws_bytes below moe_workspace_size() */
  MOE_E_HIP = -4          /* the HIP runtime reported a launch error */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_F16 = 2 } moe_dtype;
typedef enum { MOE_WF_DENSE = 0, MOE_WF_AFFINE_Q4 = 1, MOE_WF_AFFINE_Q8 = 2 } moe_wformat;
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GEGLU = 1 } moe_activation;

/*
 * Layer shape and format.
 *  d_model, d_ff  > 0; for the affine formats multiples of 64 and of
 *                 group_size (the groups run along both reduction dims);
 *                 multiples of 8 otherwise.
 *  n_experts      routed experts E, 1..1024.
 *  top_k          1..min(32, n_experts).
 *  n_shared       always-on shared experts (weight 1.0, not renormalised), 0..8;
 *                 their weights follow the E routed experts in every projection.
 *  act_dtype      moe_dtype of x, W_router and dense expert weights (fp32,
 *                 bf16 or fp16: "SwitchGLU: grouped-expert Metal kernels",
 *                 "When it applies"; DS4Server #112, "Current upstream route").
 *  w_format       moe_wformat of the expert weights.  The affine formats
 *                 (4- or 8-bit codes: "perf(moe): fused MoE expert decode
 *                 kernel", "Multi-bit handling"; DS4Server #112, "Native
 *                 implementation scope") need a 16-bit act_dtype (bf16 or
 *                 fp16); their scales and biases are in that dtype.
 *  group_size     affine group length along the reduction dim: 32, 64 or 128.
 *  gate_up_fused  1: one [2*d_ff][d_model] matrix per expert whose rows are
 *                 [gate | up]; 0: separate gate and up matrices.
 *  glu_round      1: per-op rounding of the gated unit to the activation
 *                 dtype (bf16 or fp16, nearest even; DS4Server #112, "Kernel
 *                 contract", SwiGLU epilogue): gate and up rounded, then
 *                 sigmoid, g*s and (g*s)*u each rounded; for GeGLU gate and
 *                 up, then gelu(g) and gelu(g)*u each rounded.  Needs a
 *                 16-bit act_dtype.
 *  renormalize    1: the k selected weights are divided by their sum.
 *  activation     moe_activation of the expert GLU: SwiGLU, h = silu(g)*u,
 *                 or GeGLU with the tanh form of GELU,
 *                 h = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u
 *                 ("SwitchGLU: grouped-expert Metal kernels", "When it
 *                 applies").
 */
typedef struct {
  int32_t d_model, d_ff, n_experts, top_k, n_shared;
  int32_t act_dtype, w_format, group_size;
  int32_t gate_up_fused, glu_round, renormalize;
  int32_t activation;
} moe_layer_desc;

/*
 * One projection for all experts (routed 0..E-1, then shared E..E+S-1), out-
 * major (the reduction dim contiguous):
 *  dense: w = act_dtype [E+S][N][K]; scales = biases = NULL.
 *  affine b-bit (b = 4 for Q4, 8 for Q8), group g:
 *         w = uint32 [E+S][N][K*b/32], column k of row n is bits
 *         [b*(k%(32/b)), +b) of word k/(32/b) (an unsigned code q in
 *         0..2^b-1); scales, biases = act_dtype (bf16 or fp16) [E+S][K/g][N] (group-major: one
 *         group's values for consecutive rows are contiguous); the weight is
 *         scale*q + bias of its group ("affine" quantisation with 16-bit scales
 *         and biases: "SwitchGLU: grouped-expert Metal kernels"
 *         (ml-explore/mlx-lm #2044), "When it applies").
 * gate, up: N = d_ff, K = d_model; gate_up: N = 2*d_ff, K = d_model;
 * down: N = d_model, K = d_ff.
 */
typedef struct {
  const void *w;
  const void *scales;
  const void *biases;
  /* Optional (NULL: none), affine formats only: the tile-packed copy that
   * moe_pack_weights writes (codes, scales and biases rearranged).  When
   * set, the grouped matrix-core kernels of moe_forward, moe_expert_ffn and
   * moe_backward read their codes from here; the forward's gate/up kernel
   * also takes its scales and group terms from it for the matrices whose
   * flag is set (see moe_pack_weights), which changes the rounding (not the
   * bound) of its results.  w, scales and biases are still required, for
   * the other kernels. */
  const void *w_packed;
} moe_proj;

typedef struct {
  const void *w_router;      /* [d_model][n_experts], act_dtype */
  const float *router_bias;  /* [n_experts] fp32 added to the logits, or NULL */
  moe_proj gate, up;         /* used when gate_up_fused == 0 */
  moe_proj gate_up;          /* used when gate_up_fused == 1 */
  moe_proj down;
  /* Optional (NULL: none): the prepared router that moe_pack_router wrote
   * from w_router.  When set, the matrix-core router (16-bit layers, T >= 64
   * with T * n_experts >= 65536) reads it instead of transposing w_router
   * on every call; routing results are the same.  It is a copy: after
   * w_router changes, write it again (a stale copy routes by the old
   * weights).  w_router is still required. */
  const void *w_router_packed;
} moe_weights;

/* Projections, for moe_packed_bytes and moe_pack_weights. */
typedef enum {
  MOE_PROJ_GATE = 0,
  MOE_PROJ_UP = 1,
  MOE_PROJ_GATE_UP = 2,
  MOE_PROJ_DOWN = 3
} moe_projection;

/*
 * Tile-packed copy of an affine projection.  The grouped kernels multiply
 * tiles of 16 weight rows and stream the reduction in slabs of 128 columns;
 * in the stored layout a slab of a tile is 16 pieces of 64 (4-bit) or 128
 * (8-bit) bytes, one per row, 1 KB or more apart.  The packed copy holds four
 * regions, each starting at a multiple of 256 bytes, in this order (M = E+S
 * matrices, N and K as in moe_proj, G = K/group_size groups per row,
 * nslab = ceil(K/128), SW = 128*b/32 words, GPS = 128/group_size,
 * GP = G rounded up to a multiple of 32, z = 8 for 4-bit and 128 for 8-bit
 * codes):
 *   codes[m][t][s][r][j] = w[m][16 t + r][SW s + j]   uint32, zero past the row;
 *   scales[m][t][s][r][i] = fp16(s), s the scale of row 16 t + r, group GPS s + i;
 *   groups[m][t][r][g]    = fp16((b - 1024 s - n2) * group_size) for row
 *                           16 t + r and group g (scale s, bias b), with
 *                           n2 = fp16(-(1024 + z) s);
 *   flags[m]  int32 1 when every scale of matrix m is 0 or an fp16 value in
 *             [2^-14, 32] and every group term is finite and below 2^15 in
 *             magnitude, else 0
 * (scales and group terms zero past the last group).  For matrices with the
 * flag set, the forward's gate/up kernel expands a code q to
 * fp16(s*(1024 + q) + n2) = fp16(s*(q - z) + delta), which is one fma and
 * keeps the rounding error of s*q + b, and adds the rest of every weight of
 * the group, b - 1024 s - n2, as one fp16 matrix-core product of the group
 * terms with the group means of x.  The sum is the same
 * (scale*q + bias) * x, rounded in other places.  The copy is an addition for
 * callers that keep a second copy of the weights (on a 288 GB device it is
 * cheap next to the time it saves).
 *
 * moe_packed_bytes: *bytes = size of the packed copy of projection `proj`
 * for all E+S matrices.  MOE_E_UNSUPPORTED for dense weights, MOE_E_INVALID
 * for a bad descriptor or a projection the descriptor does not use.
 * moe_pack_weights: enqueue the packing of `w`, `scales` and `biases`
 * (device, the stored layouts of that projection) into `w_packed` (device,
 * moe_packed_bytes bytes, 16-byte aligned) on `stream`; no host wait, no
 * allocation.  MOE_E_INVALID for a null or misaligned pointer.
 */
int moe_packed_bytes(const moe_layer_desc *desc, int32_t proj, size_t *bytes);
int moe_pack_weights(const moe_layer_desc *desc, int32_t proj, const void *w, const void *scales,
                     const void *biases, void *w_packed, void *stream);

/*
 * Prepared router ("MoE Optimization COMPLETE", "Optimization Technique": the
 * router matmul on the GPU).  The matrix-core router multiplies the rows of
 * the transposed router weight and bounds its rounding with the experts'
 * weight norms; both depend on the weights only, so a caller whose router
 * does not change can prepare them once.  The prepared router holds
 *   wt[e][i]   = w_router[i][e], act_dtype, [n_experts][d_model];
 *   then, from a multiple of 256 bytes, normp[kb][e] = sum of squares of
 *   w_router[256 kb .. 256 kb + 255][e] (fp32, kb < ceil(d_model/256)), and
 *   norms[e] = those partials summed in kb order (fp32).
 * moe_router_packed_bytes: *bytes = its size; MOE_E_UNSUPPORTED for fp32
 * layers and for d_model not a multiple of 64 or above 4096 (the layers the
 * matrix-core router does not take), MOE_E_INVALID for a bad descriptor.
 * moe_pack_router: enqueue its writing from `w_router` (device) into `out`
 * (device, moe_router_packed_bytes bytes, 16-byte aligned) on `stream`; no
 * host wait, no allocation; MOE_E_INVALID for a null or misaligned pointer.
 * The copy does not follow later changes to w_router: write it again after
 * each change, before the next call that is given it.
 */
int moe_router_packed_bytes(const moe_layer_desc *desc, size_t *bytes);
int moe_pack_router(const moe_layer_desc *desc, const void *w_router, void *out, void *stream);

/* Bytes of workspace that moe_dispatch, moe_expert_ffn and moe_forward need
 * for this layer at T tokens (also valid for any smaller T).  Returns
 * MOE_E_INVALID for a bad descriptor or T < 0. */
int moe_workspace_size(const moe_layer_desc *desc, int32_t T, size_t *bytes);

/*
 * Router (step 1): topk_idx[T][k] int32 and topk_w[T][k] fp32 from x[T][d_model]
 * and w_router[d_model][E] (+ router_bias[E] or NULL).  Logits use a fixed
 * fp32 order: per (t, e), chunks of 64 consecutive columns, each chunk a
 * sequential fma chain from +0, chunk sums added in ascending order from +0,
 * bias added last.  Slot j holds the j-th largest logit (ties to the lower
 * expert index); the weights are the fp32 softmax over all E logits, divided
 * by their sum over the k slots when renormalize is set.  The logits live in
 * the workspace (sized by moe_workspace_size); they are not an output.
 */
int moe_route(const moe_layer_desc *desc, int32_t T, const void *x,
              const void *w_router, const float *router_bias,
              int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              void *stream);

/*
 * Dispatch (step 2, DS4Server #112 "Current upstream route", sort_rows, and
 * "Kernel contract", per-expert tile/row prefix tables): for the N = T*k flat
 * slots i = t*k + j with expert f[i] = topk_idx[i]:
 *   order[N]      stable argsort of f (equal experts keep ascending i);
 *   inv_order[N]  inverse permutation, inv_order[order[p]] = p;
 *   row_map[N]    order[p] / k, the token whose row sorted position p reads;
 *   expert_off[E+1]  first sorted position of each expert, expert_off[E] = N;
 *   tile_off[E+1] prefix sum of ceil(count_e / tile_rows), tile_rows >= 1.
 * All int32.  Every topk_idx entry must lie in [0, E); the kernel checks it
 * and an out-of-range entry yields order = inv_order = row_map = -1 and
 * expert_off[E] = -1 rather than an out-of-bounds write.
 */
int moe_dispatch(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                 int32_t tile_rows, int32_t *order, int32_t *inv_order,
                 int32_t *row_map, int32_t *expert_off, int32_t *tile_off,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Grouped expert FFN (step 3): for sorted routed row p < N (expert e with
 * expert_off[e] <= p < expert_off[e+1], token row_map[p]) and shared row
 * p = N + s*T + t (shared expert s, token t):
 *   y_sorted[p][:] = down_e( SwiGLU( gate_e . x[token], up_e . x[token] ) ),
 * fp32, y_sorted [N + n_shared*T][d_model].  row_map and expert_off are as
 * moe_dispatch writes them.
 */
int moe_expert_ffn(const moe_layer_desc *desc, int32_t T, const void *x,
                   const int32_t *row_map, const int32_t *expert_off,
                   const moe_weights *w, float *y_sorted, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * Combine (step 4, DS4Server #112 "_scatter_unsort" through inv_order):
 *   y[t][:] = sum_{j<k} topk_w[t][j] * y_sorted[inv_order[t*k+j]][:]
 *             + sum_{s<n_shared} y_sorted[N + s*T + t][:],
 * accumulated in fp32 in that order, then stored as out_dtype (moe_dtype;
 * bf16 and fp16 round to nearest even once).
 */
int moe_combine(const moe_layer_desc *desc, int32_t T, const float *y_sorted,
                const int32_t *inv_order, const float *topk_w, void *y,
                int32_t out_dtype, void *stream);

/*
 * The whole layer (steps 1-4) in one call, all on `stream`.  y[T][d_model] in
 * out_dtype.  topk_idx_out[T][k] / topk_w_out[T][k] receive the routing when
 * non-NULL.  Routing and dispatch results equal those of moe_route and
 * moe_dispatch bit for bit.
 */
int moe_forward(const moe_layer_desc *desc, int32_t T, const void *x,
                const moe_weights *w, void *y, int32_t out_dtype,
                int32_t *topk_idx_out, float *topk_w_out, void *ws,
                size_t ws_bytes, void *stream);

/*
 * moe_forward for profiling: the same work, with kernel i of the call (in
 * launch order) launched through hipExtLaunchKernel with events[2i] and
 * events[2i+1] as its start and stop events, for as many kernels as
 * n_events / 2 covers (hipEvent_t handles created by the caller; kernels past
 * them launch plainly).  The elapsed time between a kernel's two events is
 * that kernel's own execution, with no launch gap inside.  names (nullable,
 * names_len bytes) receives one comma-separated stage name per kernel, in
 * launch order, truncated to fit (a stage such as "dispatch" or "route_mfma"
 * may run two kernels).  Only the calling host thread's launches inside this
 * call are affected.
 */
int moe_forward_timed(const moe_layer_desc *desc, int32_t T, const void *x,
                      const moe_weights *w, void *y, int32_t out_dtype,
                      int32_t *topk_idx_out, float *topk_w_out, void *ws,
                      size_t ws_bytes, void *stream, void *const *events,
                      int32_t n_events, char *names, size_t names_len);

/*
 * Backward of the layer with respect to x ("SwitchGLU: grouped-expert Metal
 * kernels", section "What": the grouped experts carry a custom VJP for
 * training through them).  dy[T][d_model] fp32 is the gradient of the loss
 * with respect to the forward's y; dx[T][d_model] fp32 receives
 * dy . dy/dx with the weights fixed and the routing held at the forward's
 * choice: through the selected experts (scaled by their weights), the shared
 * experts, and the softmax (renormalised or not) that gives the slot weights,
 * then W_router.  The forward's per-op rounding is not differentiated.  The
 * router and dispatch run again inside.  fp32 layers compute in fp32 on the
 * vector units; 16-bit layers run the contractions on the matrix cores (the
 * gate/up recomputation as in the forward; the transposed products on fp16
 * operands with power-of-two exponents, or for dense bf16 weights on the
 * exact weights against a bf16 head/tail split of the activations; fp32
 * accumulation).  Repeated calls give identical bits.
 * ws: moe_backward_workspace_size bytes (caller-owned, 16-byte aligned).
 * Errors as for moe_forward.
 */
int moe_backward_workspace_size(const moe_layer_desc *desc, int32_t T, size_t *bytes);
int moe_backward(const moe_layer_desc *desc, int32_t T, const void *x,
                 const moe_weights *w, const float *dy, float *dx, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call itself allocates nothing.  Layers whose
 * moe_workspace_size(desc, T) exceeds MOE_NOALLOC_SCRATCH_BYTES get
 * MOE_E_WORKSPACE and nothing is enqueued (the one-token and 32-token decode
 * layers need well under 8 MiB, a 512-token dense layer with 8 experts about
 * 75 MiB).  The work runs on the device current at the call, which must be
 * the device of `stream`.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (other streams, other host threads) race:
 * serialise them.  Other arguments and results as for moe_forward.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
int moe_forward_noalloc(const moe_layer_desc *desc, int32_t T, const void *x,
                        const moe_weights *w, void *y, int32_t out_dtype,
                        int32_t *topk_idx_out, float *topk_w_out, void *stream);

/*
 * A plain streaming read, outside the layer: the rate a kernel of this
 * library reaches when it only reads, the scale for the HBM rooflines of the
 * weight-streaming kernels.  blocks workgroups of 256 threads read the
 * `bytes` at src (device memory, 16-byte aligned, bytes a multiple of 16)
 * with 16-byte loads, grid-stride, and each thread writes the XOR of the
 * words it read to out[blocks * 256] (device memory, caller-owned).  Enqueued
 * on `stream`; MOE_E_INVALID for a null pointer, a misaligned src, a size
 * that is 0 or not a multiple of 16, or blocks outside [1, 65536];
 * MOE_E_HIP if the launch fails.
 */
int moe_stream_read(const void *src, size_t bytes, uint32_t *out, int32_t blocks, void *stream);

/* A static, human-readable name of a moe_status value. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
