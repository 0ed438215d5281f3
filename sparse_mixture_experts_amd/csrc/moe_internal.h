// moe_internal.h -- host-side plumbing shared by the library's translation
// units: descriptor validation, workspace layout and kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_mi355x.h"

namespace moe {

// One unit of expert work: `rows` consecutive sorted rows starting at `row0`,
// all routed to `expert` (shared experts have ids E..E+S-1).
struct PlanItem {
  int32_t expert, row0, rows, pad;
};

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 8;
constexpr int kMinTileRows = 16;  // smallest row tile of the grouped MFMA kernels

// Host-side checks (no HIP calls); return a moe_status.
int validate_desc(const moe_layer_desc *d);
int validate_T(int32_t T);
int validate_ptr(const void *p, bool may_be_null = false);
int validate_weights(const moe_layer_desc *d, const moe_weights *w, bool need_router,
                     bool need_experts);

inline int64_t act_bytes(const moe_layer_desc *d) { return d->act_dtype == MOE_DT_F32 ? 4 : 2; }
// Affine 4- or 8-bit expert weights (fp16 matrix-core path with fp16 staging).
inline bool affine(const moe_layer_desc *d) {
  return d->w_format == MOE_WF_AFFINE_Q4 || d->w_format == MOE_WF_AFFINE_Q8;
}
// Bytes per element of the GLU intermediate h (16-bit for bf16 and fp16 layers).
inline int64_t h_bytes(const moe_layer_desc *d) { return d->act_dtype == MOE_DT_F32 ? 4 : 2; }
bool use_mfma(const moe_layer_desc *d);

// Workspace carve-up.  Every section is 256-byte aligned.
struct Workspace {
  size_t topk_idx, topk_w;            // [N] int32 / f32 (moe_forward without caller buffers)
  size_t route;                       // router logits / chunk partials (f32)
  size_t order, inv_order, row_map;   // [N] int32
  size_t expert_off, tile_off;        // [E+1] int32
  size_t counters;                    // 64 int32: [0] active items, [1] tiles
  size_t dsp;                         // dispatch scratch (dispatch_scratch_ints)
  size_t act_items;                   // [E+S] PlanItem
  size_t tiles;                       // [max_tiles] PlanItem
  size_t h;                           // [N+S*T][d_ff] h_bytes
  size_t hsh;                         // [N+S*T][ceil(d_ff/128)] int8 (affine layers)
  size_t x16, xsh;                    // [T][d_model] fp16, [T] int8 (affine layers)
  size_t y_sorted;                    // [N+S*T][d_model]: fp16 (ys_f16e), fp32, or [parts] fp32 partial rows
  size_t ys_sh;                       // [N+S*T][d_model/64] int8 exponents (ys_f16e)
  size_t total;
  int64_t max_tiles;
};
Workspace workspace_layout(const moe_layer_desc *d, int32_t T);

// Optional hook called after each kernel launch (profiling builds of the
// forward pass record a stream event there).
struct StageMarker {
  virtual void mark(const char *stage) = 0;
  virtual ~StageMarker() = default;
};

// ---- launchers (defined next to their kernels; all asynchronous) ----------

// Router: topk idx/w for T tokens; scratch holds route_scratch_floats floats.
int64_t route_scratch_floats(const moe_layer_desc *d, int32_t T);
// Matrix-core router with exact recomputation of the candidates (large T).
bool route_mfma_applies(const moe_layer_desc *d, int32_t T);
int64_t route_mfma_scratch_floats(const moe_layer_desc *d, int32_t T);
void launch_route_mfma(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router, const float *bias,
                       int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh, void *stream,
                       StageMarker *mk);
// Outputs of a dispatch that the router's selection kernel performs itself
// (order == nullptr: none).
struct FusedDispatch {
  int32_t *order, *inv_order, *row_map, *expert_off, *tile_off, *counters;
  PlanItem *act_items, *tiles;
  int tile_rows, tr, S;
};
// x16/xsh (nullable): the router's per-token kernel also writes the fp16
// staging copy of x for the 4-bit GEMMs when route_writes_x16 holds.  With
// dsp.order set and route_fuses_dispatch true it also does the dispatch.
bool route_writes_x16(const moe_layer_desc *d);
bool route_fuses_dispatch(const moe_layer_desc *d, int32_t T);
void launch_route(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router,
                  const float *bias, int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh,
                  const FusedDispatch &dsp, void *stream, StageMarker *mk = nullptr);

// Dispatch: stable counting sort + prefix tables + the internal work plan.
// scratch holds dispatch_scratch_ints ints (per-workgroup counts for large N).
int64_t dispatch_scratch_ints(const moe_layer_desc *d, int32_t T);
void launch_dispatch(const moe_layer_desc *d, int32_t T, const int32_t *idx, int32_t tile_rows,
                     int32_t *order, int32_t *inv_order, int32_t *row_map, int32_t *expert_off,
                     int32_t *tile_off, int32_t *counters, PlanItem *act_items, PlanItem *tiles,
                     int32_t *scratch, void *stream, StageMarker *mk = nullptr);

// Work plan from caller-supplied expert offsets (standalone moe_expert_ffn).
void launch_plan(const moe_layer_desc *d, int32_t T, const int32_t *expert_off, int32_t *counters,
                 PlanItem *act_items, PlanItem *tiles, void *stream);

// Intermediate buffers of the expert FFN (all in the workspace).  h holds
// the SwiGLU rows; on the 4-bit matrix-core path h is fp16 with a power-of-two
// exponent per (row, 128-column block) in hsh, and x16/xsh hold the fp16 copy
// of x with one exponent per token.
struct FfnScratch {
  void *h;
  int8_t *hsh;
  void *x16;
  int8_t *xsh;
  bool x16_ready;  // x16/xsh already written (by the router)
};
constexpr int kHBlock = 128;  // h columns per exponent block

// Reduction parts of the down projection inside moe_forward (1: none).  With
// more, the expert outputs are fp32 partial rows [parts][N+S*T][d_model]
// that the combine adds in part order.
int ffn_down_parts(const moe_layer_desc *d, int32_t T);
// Expert outputs inside moe_forward as fp16 values v with one power-of-two
// exponent e per (row, 64 columns), y = v * 2^e: on the 16-bit matrix-core
// tiles when the down reduction is not split.  Otherwise fp32.
bool ys_f16e(const moe_layer_desc *d, int32_t T);
// Workspace bytes for the expert outputs of any call with at most T tokens.
int64_t ys_workspace_bytes(const moe_layer_desc *d, int32_t T);
constexpr int kYsBlock = 64;  // expert-output columns per exponent

// Expert FFN over the plan: y_sorted rows for all routed and shared rows,
// fp32 (ys_sh null), fp16 with exponents in ys_sh (ys_f16e layers), or fp32
// partial rows (down_parts > 1).
void launch_expert_ffn(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                       const moe_weights *w, const int32_t *counters, const PlanItem *act_items,
                       const PlanItem *tiles, int64_t max_tiles, const FfnScratch &sc, void *y_sorted,
                       int8_t *ys_sh, void *stream, StageMarker *mk = nullptr, int down_parts = 1);

// Row-tile height of the work plan for this layer and token count, and
// whether the grouped MFMA kernels serve the layer (else dequant-GEMV).
int plan_tile_rows(const moe_layer_desc *d, int32_t T);
void launch_expert_ffn_mfma(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                            const moe_weights *w, const int32_t *counters, const PlanItem *tiles,
                            int64_t max_tiles, const FfnScratch &sc, void *y_sorted, int8_t *ys_sh, void *stream,
                            StageMarker *mk, int down_parts = 1);

// Backward with respect to x.  Intermediates in the backward workspace (R
// sorted rows): g and u, v = Wd^T dy (per reduction split), dw, the rows'
// dx (per split), the router matrix transposed for the per-token kernel;
// the matrix-core path adds dg | du as bf16.
struct BwdScratch {
  float *gu;      // matrix cores: [R][2F] g | u per row; vector units: g [R][F] then u [R][F]
  float *v;       // [splits.v][R][F]
  float *dw;      // [R]
  float *dxr;     // [splits.dx][R][D]
  uint16_t *dgu;  // matrix-core path: [R][2F] bf16, dg then du
  void *wr_t;     // router matrix transposed [E][D] (layer dtype)
  FfnScratch ffn; // matrix-core path: the fp16 staging copy of x (affine layers)
};
// Reduction splits of the matrix-core backward's transposed products (the
// partial sums are added in split order by their consumers).
struct BwdSplits {
  int v, dx;
};
BwdSplits backward_splits(const moe_layer_desc *d, int32_t T);
struct BwdWorkspace {
  Workspace fwd;  // router and dispatch sections (the forward's layout)
  size_t gu, v, dw, dxr, dgu, wr_t, total;
};
BwdWorkspace backward_workspace_layout(const moe_layer_desc *d, int32_t T);
void launch_backward(const moe_layer_desc *d, int32_t T, const void *x, const moe_weights *w, const float *dy,
                     const int32_t *topk_idx, const float *topk_w, const int32_t *order, const int32_t *inv_order,
                     const int32_t *row_map, const int32_t *counters, const PlanItem *items, const PlanItem *tiles,
                     int64_t max_tiles, const BwdScratch &sc, float *dx, void *stream);
// Matrix-core part of the backward (16-bit layers): sc.dw and sc.dxr.
void launch_backward_mfma(const moe_layer_desc *d, int32_t T, const void *x, const moe_weights *w, const float *dy,
                          const float *topk_w, const int32_t *order, const int32_t *row_map,
                          const int32_t *counters, const PlanItem *tiles, int64_t max_tiles, const BwdScratch &sc,
                          void *stream);
// The grouped gate/up GEMM without the GLU: gu[r] = [x Wg^T | x Wu^T] for
// every sorted row r (fp32, row stride 2*d_ff), x read through row_map as in
// the forward (the fp16 staging copy for affine layers, written here unless
// sc.x16_ready).
void launch_gate_up_raw_mfma(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                             const moe_weights *w, const int32_t *counters, const PlanItem *tiles, int64_t max_tiles,
                             const FfnScratch &sc, float *gu, void *stream);

// Combine.
// Combine of fp32 rows (ys_sh null), fp16 rows with exponents ys_sh, or
// parts > 1 fp32 partial rows added in part order.
void launch_combine(const moe_layer_desc *d, int32_t T, const void *y_sorted, const int8_t *ys_sh,
                    const int32_t *inv_order, const float *topk_w, void *y, int32_t out_dtype,
                    void *stream, StageMarker *mk = nullptr, int parts = 1);

}  // namespace moe
