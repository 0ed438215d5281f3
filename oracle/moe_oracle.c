/*
 * moe_oracle.c -- plain, slow, obviously correct CPU reference for the
 * sparse MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code
 * with the GPU library.  Build: gcc -O2 -ffp-contract=off -fopenmp (no
 * fast-math), so every fp32 operation below happens as written.
 *
 * Pins: every function here is checked by the CPU tests against something
 * other than itself (NumPy fp64 brute force on small shapes, closed forms,
 * invariants, torch's bf16 cast); see the header of each test file.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t g_last_threads = 1;

/* bf16 <-> fp32.  Widening is exact (the bf16 bits are the top half of the
 * fp32 bits).  Narrowing rounds to nearest, ties to even, and keeps NaN
 * quiet. */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static float round_bf16(float f) { return oracle_bf16_to_f32(oracle_f32_to_bf16(f)); }

/* IEEE binary16 -> fp32, exact: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 holds subnormals (fraction * 2^-24), 31 infinities and
 * NaNs. */
float oracle_f16_to_f32(uint16_t h) {
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 0x400u), (int)e - 25);
  return (h & 0x8000u) ? -v : v;
}

/* fp32 -> IEEE binary16, round to nearest, ties to even.  The value is
 * scaled into binary16's grid by its exponent: normal results keep 11
 * significant bits (1 implicit + 10 stored), results below 2^-14 are
 * multiples of 2^-24 (subnormals), results at or above 65520 overflow to
 * infinity; NaN stays a quiet NaN.  The rounding is done on the exact fp32
 * bits: the kept part and the discarded remainder are compared with half a
 * unit of the last kept place. */
uint16_t oracle_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t ex = (u >> 23) & 0xffu, man = u & 0x7fffffu;
  if (ex == 0xffu) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u)); /* inf / NaN */
  if (ex == 0 && man == 0) return sign;                                   /* +-0 (fp32 subnormals below too) */
  /* the value is sig * 2^(e - 23) with sig the 24-bit significand */
  const uint32_t sig = ex ? (man | 0x800000u) : man;
  const int32_t e = ex ? (int32_t)ex - 127 : -126;
  /* binary16 keeps bits down to 2^(max(e, -14) - 10): drop `sh` low bits of sig */
  const int32_t keep_exp = (e < -14 ? -14 : e) - 10;
  const int32_t sh = keep_exp - (e - 23);
  uint32_t q;
  if (sh >= 32) {
    q = 0; /* far below half of the smallest subnormal */
  } else {
    q = sig >> sh;
    const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
  }
  /* q counts units of 2^keep_exp; rebuild the binary16 fields */
  if (e < -14) return (uint16_t)(sign | q); /* subnormal (q = 1024 carries into the smallest normal) */
  int32_t be = e + 15;
  if (q == 2048u) { /* rounding carried into the next binade */
    q = 1024u;
    be += 1;
  }
  if (be >= 31) return (uint16_t)(sign | 0x7c00u); /* overflow */
  return (uint16_t)(sign | ((uint32_t)be << 10) | (q & 0x3ffu));
}

static float round_f16(float f) { return oracle_f16_to_f32(oracle_f32_to_f16(f)); }

/* Per-op rounding of the gated epilogue to the layer's 16-bit activation
 * dtype (DS4Server #112, "Kernel contract": the SwiGLU accumulators are
 * rounded to the activation dtype, bf16 or fp16). */
static float round_act(const oracle_desc *d, float f) { return d->act_f16 ? round_f16(f) : round_bf16(f); }

/* A 16-bit value of the activation dtype (bf16, or fp16 with act_f16). */
static float half_at(const oracle_desc *d, uint16_t h) {
  return d->act_f16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

/* Element i of an activation-dtype array. */
static float act_at(const oracle_desc *d, const void *p, int64_t i) {
  if (d->act_bf16 || d->act_f16) return half_at(d, ((const uint16_t *)p)[i]);
  return ((const float *)p)[i];
}

/*
 * Router logits.  The pages put router matmul, softmax and top-K on the GPU
 * with no host round trip ("MoE Optimization COMPLETE", section "Mega Kernel
 * Architecture": router matmul, softmax, top-K phases; PRD "5.5 real sparse
 * MoE kernels (Metal)", section "Scope - in": top-K routing kernel).  They do
 * not fix the fp32 accumulation order, yet expert indices must agree bit for
 * bit between implementations, so one order is fixed here (the canonical
 * order):
 *   the reduction over d runs in chunks of 64 consecutive columns; inside a
 *   chunk a partial p starts at +0 and takes p = fma(x[i], W[i][e], p) for i
 *   ascending; the chunk partials are added to an accumulator that starts at
 *   +0, chunk by chunk in ascending order; the optional fp32 router bias is
 *   added last.
 */
void oracle_router_logits(const oracle_desc *d, int32_t T, const void *x,
                          const void *w_router, const float *router_bias,
                          float *logits) {
  const int32_t D = d->d_model, E = d->n_experts;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t c0 = 0; c0 < D; c0 += 64) {
        int32_t c1 = c0 + 64 < D ? c0 + 64 : D;
        float p = 0.0f;
        for (int32_t i = c0; i < c1; ++i)
          p = fmaf(act_at(d, x, (int64_t)t * D + i),
                   act_at(d, w_router, (int64_t)i * E + e), p);
        acc = acc + p;
      }
      if (router_bias) acc = acc + router_bias[e];
      logits[(int64_t)t * E + e] = acc;
    }
  }
}

/* a ranks before b: larger logit first; equal logits (IEEE equality, so
 * -0 == +0) go to the lower expert index. */
static int ranks_before(float la, int32_t a, float lb, int32_t b) {
  if (la > lb) return 1;
  if (la < lb) return 0;
  return a < b;
}

/*
 * Selection and weights for one token: the top_k experts in descending logit
 * order with lowest-index tie-break (slot j holds the j-th of them), then
 * softmax over all E logits in fp32 (max subtracted, exponentials summed in
 * ascending expert order) and, if requested, renormalisation of the selected
 * probabilities (summed in slot order) so they add to one.  Selection works
 * on logits: softmax is increasing, so the selected set is the same, and
 * rounding in expf cannot merge two distinct logits into a tie.
 */
static void route_one(const oracle_desc *d, const float *l, int32_t *idx,
                      float *w) {
  const int32_t E = d->n_experts, K = d->top_k;
  char *taken = (char *)calloc((size_t)E, 1);
  for (int32_t j = 0; j < K; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
  free(taken);

  float m = l[0];
  for (int32_t e = 1; e < E; ++e)
    if (l[e] > m) m = l[e];
  float z = 0.0f;
  for (int32_t e = 0; e < E; ++e) z = z + expf(l[e] - m);
  float psum = 0.0f;
  for (int32_t j = 0; j < K; ++j) {
    w[j] = expf(l[idx[j]] - m) / z;
    psum = psum + w[j];
  }
  if (d->renormalize)
    for (int32_t j = 0; j < K; ++j) w[j] = w[j] / psum;
}

void oracle_route(const oracle_desc *d, int32_t T, const void *x,
                  const void *w_router, const float *router_bias,
                  int32_t *topk_idx, float *topk_w) {
  const int32_t E = d->n_experts, K = d->top_k;
  const size_t row_bytes = (size_t)d->d_model * (d->act_bf16 || d->act_f16 ? 2 : 4);
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    float *l = (float *)malloc(sizeof(float) * (size_t)E);
    oracle_router_logits(d, 1, (const char *)x + (size_t)t * row_bytes,
                         w_router, router_bias, l);
    route_one(d, l, topk_idx + (int64_t)t * K, topk_w + (int64_t)t * K);
    free(l);
  }
}

/*
 * Dispatch (DS4Server issue #112, "Current upstream route", sort_rows):
 * flat slot i = t*k + j carries expert f[i] = topk_idx[t][j];
 * order = argsort(f), stable (equal experts keep ascending slot order);
 * inv_order = argsort(order), i.e. inv_order[order[p]] = p;
 * row_map[p] = order[p] / k (the token whose row sorted position p reads).
 * Per-expert prefix tables ("Kernel contract": per-expert tile/row prefix
 * tables): expert_off[e] = number of slots routed to experts < e;
 * tile_off[e] = sum over experts < e of ceil(count / tile_rows).
 */
static const int32_t *g_sort_keys;
static int cmp_slot(const void *a, const void *b) {
  int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  if (g_sort_keys[i] != g_sort_keys[j]) return g_sort_keys[i] < g_sort_keys[j] ? -1 : 1;
  return i < j ? -1 : (i > j);
}

void oracle_dispatch(int32_t T, int32_t top_k, int32_t n_experts,
                     const int32_t *topk_idx, int32_t tile_rows,
                     int32_t *order, int32_t *inv_order, int32_t *row_map,
                     int32_t *expert_off, int32_t *tile_off) {
  const int32_t N = T * top_k;
  for (int32_t i = 0; i < N; ++i) order[i] = i;
  g_sort_keys = topk_idx;
  qsort(order, (size_t)N, sizeof(int32_t), cmp_slot);
  for (int32_t p = 0; p < N; ++p) {
    inv_order[order[p]] = p;
    row_map[p] = order[p] / top_k;
  }
  for (int32_t e = 0; e <= n_experts; ++e) expert_off[e] = 0;
  for (int32_t i = 0; i < N; ++i) expert_off[topk_idx[i] + 1] += 1;
  tile_off[0] = 0;
  for (int32_t e = 0; e < n_experts; ++e) {
    int32_t cnt = expert_off[e + 1];
    tile_off[e + 1] = tile_off[e] + (cnt + tile_rows - 1) / tile_rows;
    expert_off[e + 1] = expert_off[e] + cnt;
  }
}

/*
 * Explicit dequantisation of one weight row.  Affine 4- or 8-bit ("perf(moe):
 * fused MoE expert decode kernel", section "Multi-bit handling": affine,
 * power-of-two bits 4/8, shift-unpack; DS4Server #112, "Native implementation
 * scope": biases present, 4 or 8 bits, group 32/64/128): w = scale * q + bias,
 * q the unsigned code of the column, scale/bias the bf16 pair of the column's
 * group.  Scales and biases are in the 16-bit activation dtype (bf16, or fp16
 * for fp16 layers: "SwitchGLU: grouped-expert Metal kernels", "When it
 * applies", and DS4Server #112, "Current upstream route", both take bf16 or
 * fp16 activations with scales in the same dtype).  The product of such a scale (at most
 * 11 significant bits) and a code of at most 8 bits is exact in fp32, so only
 * the addition rounds.
 */
void oracle_dequant_row(const oracle_desc *d, const oracle_proj *p, int32_t e,
                        int32_t n, int32_t N, int32_t K, float *out) {
  if (!d->w_q4) {
    const int64_t base = ((int64_t)e * N + n) * K;
    for (int32_t k = 0; k < K; ++k) out[k] = act_at(d, p->w, base + k);
    return;
  }
  const int32_t G = d->group_size;
  const int32_t bits = d->w_bits ? d->w_bits : 4;
  const int32_t per = 32 / bits;              /* codes per word */
  const uint32_t mask = (1u << bits) - 1u;
  const uint32_t *wq = (const uint32_t *)p->w + ((int64_t)e * N + n) * (K / per);
  /* scales/biases are group-major: [expert][group][row] */
  const uint16_t *sc = p->scales + (int64_t)e * (K / G) * N + n;
  const uint16_t *bi = p->biases + (int64_t)e * (K / G) * N + n;
  for (int32_t k = 0; k < K; ++k) {
    uint32_t q = (wq[k / per] >> (bits * (k % per))) & mask;
    float s = half_at(d, sc[(int64_t)(k / G) * N]);
    float b = half_at(d, bi[(int64_t)(k / G) * N]);
    out[k] = s * (float)q + b;
  }
}

static float silu(float g) { return g / (1.0f + expf(-g)); }
static float sigmoid(float g) { return 1.0f / (1.0f + expf(-g)); }
/* tanh approximation of GELU: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) */
static float gelu_tanh(float g) {
  const float c = 0.7978845608028654f;
  return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
}

/*
 * One expert on one token (e may name a shared expert: e >= E).
 * gate/up: g[n] = sum_k x[k] * Wg[n][k], u[n] likewise, fp32, k ascending.
 * SwiGLU: h = silu(g) * u in fp32; with per-op bf16 rounding (DS4Server #112,
 * "Kernel contract", SwiGLU epilogue: accumulators rounded to the activation
 * dtype, then sigmoid and each multiply rounded as separate ops):
 *   g, u <- bf16(g), bf16(u); s = bf16(sigmoid(g)); a = bf16(g*s); h = bf16(a*u).
 * GeGLU ("SwitchGLU: grouped-expert Metal kernels", "When it applies":
 * SwiGLU or tanh-GELU GLU): h = gelu_tanh(g) * u; with per-op rounding
 *   g, u <- bf16(g), bf16(u); a = bf16(gelu_tanh(g)); h = bf16(a*u).
 * down: out[m] = sum_n h[n] * Wd[m][n], fp32, n ascending.
 * The fused [gate | up] matrix holds gate in rows 0..d_ff-1 and up in rows
 * d_ff..2*d_ff-1.
 */
/* Row n of expert e's gate and up matrices, dequantised.  The fused
 * [gate | up] matrix holds gate in rows 0..d_ff-1 and up in rows
 * d_ff..2*d_ff-1. */
static void gate_row(const oracle_desc *d, const oracle_experts *w, int32_t e, int32_t n, float *row) {
  const int32_t D = d->d_model, F = d->d_ff;
  if (d->gate_up_fused)
    oracle_dequant_row(d, &w->gate_up, e, n, 2 * F, D, row);
  else
    oracle_dequant_row(d, &w->gate, e, n, F, D, row);
}
static void up_row(const oracle_desc *d, const oracle_experts *w, int32_t e, int32_t n, float *row) {
  const int32_t D = d->d_model, F = d->d_ff;
  if (d->gate_up_fused)
    oracle_dequant_row(d, &w->gate_up, e, F + n, 2 * F, D, row);
  else
    oracle_dequant_row(d, &w->up, e, n, F, D, row);
}

void oracle_expert_apply(const oracle_desc *d, const oracle_experts *w,
                         int32_t e, const void *x_row, float *h_out,
                         float *out) {
  const int32_t D = d->d_model, F = d->d_ff;
  float *xr = (float *)malloc(sizeof(float) * (size_t)D);
  float *row = (float *)malloc(sizeof(float) * (size_t)(D > F ? D : F));
  float *h = (float *)malloc(sizeof(float) * (size_t)F);
  for (int32_t k = 0; k < D; ++k) xr[k] = act_at(d, x_row, k);

  for (int32_t n = 0; n < F; ++n) {
    float g = 0.0f, u = 0.0f;
    gate_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) g = g + xr[k] * row[k];
    up_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) u = u + xr[k] * row[k];
    if (d->activation == 1) {
      if (d->glu_round) {
        g = round_act(d, g);
        u = round_act(d, u);
        h[n] = round_act(d, round_act(d, gelu_tanh(g)) * u);
      } else {
        h[n] = gelu_tanh(g) * u;
      }
    } else if (d->glu_round) {
      g = round_act(d, g);
      u = round_act(d, u);
      float s = round_act(d, sigmoid(g));
      float a = round_act(d, g * s);
      h[n] = round_act(d, a * u);
    } else {
      h[n] = silu(g) * u;
    }
  }
  for (int32_t m = 0; m < D; ++m) {
    oracle_dequant_row(d, &w->down, e, m, D, F, row);
    float o = 0.0f;
    for (int32_t n = 0; n < F; ++n) o = o + h[n] * row[n];
    out[m] = o;
  }
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)F);
  free(xr);
  free(row);
  free(h);
}

/*
 * Layer forward for selected tokens.  For token t: route, then for each slot
 * j in order y += w[t][j] * expert_{idx[t][j]}(x[t]) (fp32, slot order), then
 * y += shared_s(x[t]) for each always-on shared expert with weight 1.0.
 * Nothing is sorted, tiled or grouped here: each selected expert is applied
 * to the token directly.
 */
void oracle_forward_tokens(const oracle_desc *d, int32_t T, const void *x,
                           const void *w_router, const float *router_bias,
                           const oracle_experts *w, int32_t n_tok,
                           const int32_t *tokens, float *y, int32_t *topk_idx,
                           float *topk_w, int32_t n_threads) {
  (void)T;
  const int32_t D = d->d_model, K = d->top_k, E = d->n_experts;
  const size_t esz = d->act_bf16 || d->act_f16 ? 2 : 4;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
  g_last_threads = omp_get_max_threads();
#else
  (void)n_threads;
  g_last_threads = 1;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < n_tok; ++r) {
    const int32_t t = tokens[r];
    const void *xt = (const char *)x + (size_t)t * D * esz;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    float *wt = (float *)malloc(sizeof(float) * (size_t)K);
    float *o = (float *)malloc(sizeof(float) * (size_t)D);
    float *yr = y + (int64_t)r * D;
    oracle_route(d, 1, xt, w_router, router_bias, idx, wt);
    for (int32_t m = 0; m < D; ++m) yr[m] = 0.0f;
    for (int32_t j = 0; j < K; ++j) {
      oracle_expert_apply(d, w, idx[j], xt, NULL, o);
      for (int32_t m = 0; m < D; ++m) yr[m] = yr[m] + wt[j] * o[m];
    }
    for (int32_t s = 0; s < d->n_shared; ++s) {
      oracle_expert_apply(d, w, E + s, xt, NULL, o);
      for (int32_t m = 0; m < D; ++m) yr[m] = yr[m] + o[m];
    }
    if (topk_idx) memcpy(topk_idx + (int64_t)r * K, idx, sizeof(int32_t) * (size_t)K);
    if (topk_w) memcpy(topk_w + (int64_t)r * K, wt, sizeof(float) * (size_t)K);
    free(idx);
    free(wt);
    free(o);
  }
}

/*
 * Backward pass (vector-Jacobian product with respect to x).  "SwitchGLU:
 * grouped-expert Metal kernels", section "What": the grouped kernels carry a
 * custom VJP (the gather_qmm math) so that training through the quantised
 * experts works.  Here, for one token with upstream gradient dy:
 *   - routing: the selected experts are held at the forward's choice (the
 *     top-k set is piecewise constant in x); the gradient flows through the
 *     selected weights w_j;
 *   - expert j (weight c = w_j; shared experts c = 1): o = Wd h, h = glu(g, u),
 *     g = Wg x, u = Wu x.  dw_j = dy . o; dh = c Wd^T dy;
 *     SwiGLU: dg = dh u s (1 + g (1 - s)), s = sigmoid(g); du = dh silu(g);
 *     GeGLU:  dg = dh u gelu'(g), du = dh gelu(g), with
 *             gelu'(g) = 0.5 (1 + tanh z) + 0.5 g (1 - tanh^2 z) z',
 *             z = a (g + b g^3), z' = a (1 + 3 b g^2);
 *     dx += Wg^T dg + Wu^T du;
 *   - router: with renormalisation w = softmax over the selected logits, so
 *     dl_j = w_j (dw_j - sum_i w_i dw_i) on the selected experts only;
 *     without it w_j = p_{e_j} (softmax over all E), dl_e = p_e (dw(e) -
 *     sum_j w_j dw_j) for every e (dw(e) = 0 off the selection);
 *     dx += W_r dl (the bias does not depend on x).
 * The forward's per-op rounding is not differentiated: g, u and h are the
 * unrounded fp32 values.  Accumulation: expert parts in slot order, then the
 * shared experts, then the router part; every sum in ascending index order.
 */
static void glu_grad(const oracle_desc *d, float g, float u, float dh, float *dg, float *du) {
  if (d->activation == 1) {
    const float a = 0.7978845608028654f, b = 0.044715f;
    const float z = a * (g + b * g * g * g);
    const float th = tanhf(z);
    const float gelu = 0.5f * g * (1.0f + th);
    const float dgelu = 0.5f * (1.0f + th) + 0.5f * g * (1.0f - th * th) * a * (1.0f + 3.0f * b * g * g);
    *dg = dh * u * dgelu;
    *du = dh * gelu;
  } else {
    const float s = 1.0f / (1.0f + expf(-g));
    *dg = dh * u * (s * (1.0f + g * (1.0f - s)));
    *du = dh * (g * s);
  }
}

/* Adds one expert's contribution c * (expert e at x_row) to dx, and returns
 * dw = dy . (expert e at x_row). */
static float expert_backward(const oracle_desc *d, const oracle_experts *w, int32_t e, const float *xr,
                             const float *dyr, float c, float *dxr) {
  const int32_t D = d->d_model, F = d->d_ff;
  float *row = (float *)malloc(sizeof(float) * (size_t)(D > F ? D : F));
  float *g = (float *)malloc(sizeof(float) * (size_t)F);
  float *u = (float *)malloc(sizeof(float) * (size_t)F);
  float *h = (float *)malloc(sizeof(float) * (size_t)F);
  float *dh = (float *)calloc((size_t)F, sizeof(float));
  for (int32_t n = 0; n < F; ++n) {
    float gn = 0.0f, un = 0.0f;
    gate_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) gn = gn + xr[k] * row[k];
    up_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) un = un + xr[k] * row[k];
    g[n] = gn;
    u[n] = un;
    h[n] = d->activation == 1 ? gelu_tanh(gn) * un : silu(gn) * un;
  }
  /* o = Wd h (for dw) and dh = c Wd^T dy, row m of Wd at a time */
  float dw = 0.0f;
  for (int32_t m = 0; m < D; ++m) {
    oracle_dequant_row(d, &w->down, e, m, D, F, row);
    float o = 0.0f;
    for (int32_t n = 0; n < F; ++n) o = o + h[n] * row[n];
    dw = dw + dyr[m] * o;
    for (int32_t n = 0; n < F; ++n) dh[n] = dh[n] + dyr[m] * row[n];
  }
  for (int32_t n = 0; n < F; ++n) {
    float dg, du;
    glu_grad(d, g[n], u[n], c * dh[n], &dg, &du);
    gate_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) dxr[k] = dxr[k] + dg * row[k];
    up_row(d, w, e, n, row);
    for (int32_t k = 0; k < D; ++k) dxr[k] = dxr[k] + du * row[k];
  }
  free(row);
  free(g);
  free(u);
  free(h);
  free(dh);
  return dw;
}

void oracle_backward_tokens(const oracle_desc *d, int32_t T, const void *x,
                            const void *w_router, const float *router_bias,
                            const oracle_experts *w, int32_t n_tok,
                            const int32_t *tokens, const float *dy, float *dx,
                            int32_t n_threads) {
  (void)T;
  const int32_t D = d->d_model, K = d->top_k, E = d->n_experts;
  const size_t esz = d->act_bf16 || d->act_f16 ? 2 : 4;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
  g_last_threads = omp_get_max_threads();
#else
  (void)n_threads;
  g_last_threads = 1;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < n_tok; ++r) {
    const int32_t t = tokens[r];
    const void *xt = (const char *)x + (size_t)t * D * esz;
    const float *dyr = dy + (int64_t)r * D;
    float *dxr = dx + (int64_t)r * D;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    float *wt = (float *)malloc(sizeof(float) * (size_t)K);
    float *dw = (float *)malloc(sizeof(float) * (size_t)K);
    float *l = (float *)malloc(sizeof(float) * (size_t)E);
    float *dl = (float *)calloc((size_t)E, sizeof(float));
    float *xr = (float *)malloc(sizeof(float) * (size_t)D);
    for (int32_t k = 0; k < D; ++k) xr[k] = act_at(d, xt, k);
    oracle_router_logits(d, 1, xt, w_router, router_bias, l);
    route_one(d, l, idx, wt);
    for (int32_t k = 0; k < D; ++k) dxr[k] = 0.0f;
    for (int32_t j = 0; j < K; ++j) dw[j] = expert_backward(d, w, idx[j], xr, dyr, wt[j], dxr);
    for (int32_t s = 0; s < d->n_shared; ++s) (void)expert_backward(d, w, E + s, xr, dyr, 1.0f, dxr);
    float dot = 0.0f;
    for (int32_t j = 0; j < K; ++j) dot = dot + wt[j] * dw[j];
    if (d->renormalize) {
      for (int32_t j = 0; j < K; ++j) dl[idx[j]] = wt[j] * (dw[j] - dot);
    } else {
      /* the softmax over all E, as route_one forms it */
      float m = l[0];
      for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      float z = 0.0f;
      for (int32_t e = 0; e < E; ++e) z = z + expf(l[e] - m);
      for (int32_t e = 0; e < E; ++e) dl[e] = -(expf(l[e] - m) / z) * dot;
      for (int32_t j = 0; j < K; ++j) dl[idx[j]] = dl[idx[j]] + wt[j] * dw[j];
    }
    for (int32_t k = 0; k < D; ++k) {
      float a = 0.0f;
      for (int32_t e = 0; e < E; ++e) a = a + act_at(d, w_router, (int64_t)k * E + e) * dl[e];
      dxr[k] = dxr[k] + a;
    }
    free(idx);
    free(wt);
    free(dw);
    free(l);
    free(dl);
    free(xr);
  }
}

int32_t oracle_last_threads(void) { return g_last_threads; }
