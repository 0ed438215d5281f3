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

// Work-plan counters (int32 in the workspace): [0] active items, [1] row
// tiles, [2] 1 when at least a quarter of the tiles belong to experts (or
// shared experts) with two or more tiles: the grouped GEMMs then order their
// work in column groups (below), so the tiles of one expert read its weights
// together and all but the first find them in L2.
__host__ __device__ inline int plan_multi_tile(int multi_tiles, int tiles) { return 4 * multi_tiles >= tiles ? 1 : 0; }

// Workgroups go to the 8 XCDs round-robin by linear id.  This maps linear
// id `lin` of `total` to a work index such that each XCD takes one
// contiguous range of work indices (ranges differ in length by at most one):
// neighbouring work that shares cache lines then shares an L2.  A bijection
// on [0, total).
__host__ __device__ inline int xcd_contiguous(int lin, int total) {
  const int xcd = lin & 7, base = total >> 3, rem = total & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + (lin >> 3);
}

// Columns blocks per group in that order.
constexpr int kColGroup = 8;

// Work item -> (row tile, column block) of a grouped GEMM with n_tiles tiles
// and nbx column blocks, in groups of gc column blocks (the last group may be
// narrower): item = ((group * n_tiles) + tile) * width + block in group.
// The workgroups that an XCD runs at once take consecutive items, so they
// cover every tile of a few experts for the same gc column blocks (the
// tiles of an expert read the same weights, the blocks of a tile stage the
// same activation rows).  gc = nbx is plain tile-major order.  Every item
// below n_tiles * nbx maps to a distinct (tile, block).
__host__ __device__ inline void item_tile_block(int item, int n_tiles, int nbx, int gc, int &tile, int &bx) {
  const int span = n_tiles * gc, full = nbx / gc, g = item / span;
  const int width = g < full ? gc : nbx - full * gc;
  const int r = item - g * span;
  tile = r / width;
  bx = g * gc + r % width;
}

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
// Rows N and reduction K of a moe_projection (false: not used by the layer).
bool proj_shape(const moe_layer_desc *d, int32_t proj, int *N, int *K);
// The tile-packed copy of one projection for all M = E+S matrices, in four
// 256-byte aligned regions (byte offsets from its start):
//   codes   [M][N/16][nslab][16][SW] uint32: the codes of each (16-row tile,
//           128-column slab) in one block (zero past the row);
//   scales  [M][N/16][nslab][16][GPS] fp16: the scale s of each (row, group
//           of the slab), converted exactly (zero past the last group);
//   groups  [M][N/16][16][GP] fp16: each row's group terms in tile blocks,
//           round((b - 1024 s - n2) * group), n2 = round(-(1024 + z) s) with
//           z = 8 (4-bit) or 128 (8-bit) (zero past the last group);
//   flags   [M] int32: 1 when every scale of the matrix is 0 or an fp16
//           value in [2^-14, 32] and every group term is finite and below
//           2^15 in magnitude before rounding.
// nslab = ceil(K/128), SW = 128*b/32, GPS = 128/group, GP = G rounded up to
// a multiple of 32 (G = K/group).  For matrices with the flag set the
// gate/up kernel expands codes to round(s (q - z) + delta) and adds the
// group terms as one fp16 matrix-core product with the group means of x.
struct PackedLayout {
  int N, K, nslab, SW, GPS, G, GP;
  size_t codes, scales, biases, flags, total;
};
bool packed_layout(const moe_layer_desc *d, int32_t proj, PackedLayout *out);
// Write the tile-packed copy of one projection (codes w[E+S][N][K*b/32],
// scales and biases [E+S][G][N]) into w_packed (see moe_pack_weights).
void launch_pack(const moe_layer_desc *d, int32_t proj, const uint32_t *w, const uint16_t *scales,
                 const uint16_t *biases, void *w_packed, void *stream);
// Group entries per token row of the x group means (G rounded up to 32).
int xg_groups_padded(const moe_layer_desc *d);
// Where the kernels that write the fp16 staging copy of x also put its group
// means, for the fast gate/up path: row t of xg (gp entries) holds, for each
// group of gs staged values, fp16(sum / gs), and zero past the last group.
// xg null: not written.
struct XgOut {
  uint16_t *xg;
  int gs, gp;
};
// The destination for this layer (xg null unless the layer is affine on the
// matrix cores and xg is given).
XgOut xg_out(const moe_layer_desc *d, uint16_t *xg);

inline int64_t act_bytes(const moe_layer_desc *d) { return d->act_dtype == MOE_DT_F32 ? 4 : 2; }
// Affine 4- or 8-bit expert weights (fp16 matrix-core path with fp16 staging).
inline bool affine(const moe_layer_desc *d) {
  return d->w_format == MOE_WF_AFFINE_Q4 || d->w_format == MOE_WF_AFFINE_Q8;
}
// Bytes per element of the GLU intermediate h (16-bit for bf16 and fp16 layers).
inline int64_t h_bytes(const moe_layer_desc *d) { return d->act_dtype == MOE_DT_F32 ? 4 : 2; }
bool use_mfma(const moe_layer_desc *d);
// Per-op GLU rounding mode of the layer: 0 none, 1 bf16, 2 fp16 (the layer's
// activation dtype).
inline int glu_round_mode(const moe_layer_desc *d) {
  return d->glu_round ? (d->act_dtype == MOE_DT_F16 ? 2 : 1) : 0;
}

// Workspace carve-up.  Every section is 256-byte aligned.
struct Workspace {
  size_t topk_idx, topk_w;            // [N] int32 / f32 (moe_forward without caller buffers)
  size_t route;                       // router logits / chunk partials (f32)
  size_t order, inv_order, row_map;   // [N] int32
  size_t expert_off, tile_off;        // [E+1] int32
  size_t counters;                    // 64 int32: [0] active items, [1] tiles, [2] multi-tile experts
  size_t dsp;                         // dispatch scratch (dispatch_scratch_ints)
  size_t act_items;                   // [E+S] PlanItem
  size_t tiles;                       // [max_tiles] PlanItem
  size_t h;                           // [N+S*T][d_ff] h_bytes (one token: [k+S][d_ff] fp32)
  size_t hsh;                         // [N+S*T][ceil(d_ff/128)] int8 (affine layers)
  size_t x16, xsh;                    // [T][d_model] fp16, [T] int8 (affine layers)
  size_t xg;                          // [T][GP] fp16 group means of x16 (affine matrix-core layers)
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
// Prepared router for the matrix-core router (moe_pack_router): whether the
// layer can use one, its size, where its norms start, and its packing.
bool router_pack_applies(const moe_layer_desc *d);
size_t router_packed_bytes(const moe_layer_desc *d);
size_t router_packed_norms_offset(const moe_layer_desc *d);
void launch_pack_router(const moe_layer_desc *d, const void *w_router, void *out, void *stream);
int64_t route_mfma_scratch_floats(const moe_layer_desc *d, int32_t T);
// counts (nullable): the dispatch's per-segment expert counts [B][E+1] for
// segments of seg slots, zeroed and then written here (integer atomics).
void launch_route_mfma(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router, const float *bias,
                       int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh, XgOut xo, void *stream,
                       StageMarker *mk, int32_t *counts = nullptr, int seg = 0, const void *packed = nullptr);
// Outputs of a dispatch that the router's selection kernel performs itself
// (order == nullptr: none).
struct FusedDispatch {
  int32_t *order, *inv_order, *row_map, *expert_off, *tile_off, *counters;
  PlanItem *act_items, *tiles;
  int tile_rows, tr, S;
  // Nullable: the multi-workgroup dispatch's per-segment expert counts
  // ([B][E+1], see dispatch_segment_slots), which the matrix-core router
  // writes with integer atomics when route_counts_dispatch holds; the
  // dispatch then skips its counting pass.
  int32_t *counts = nullptr;
};
// x16/xsh (nullable): the router's per-token kernel also writes the fp16
// staging copy of x for the 4-bit GEMMs when route_writes_x16 holds.  With
// dsp.order set and route_fuses_dispatch true it also does the dispatch.
bool route_writes_x16(const moe_layer_desc *d);
bool route_fuses_dispatch(const moe_layer_desc *d, int32_t T);
// xg (nullable): the group means of the staging rows go there too.
void launch_route(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router,
                  const float *bias, int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh,
                  uint16_t *xg, const FusedDispatch &dsp, void *stream, StageMarker *mk = nullptr,
                  const void *router_packed = nullptr);

// One-token router logits as canonical-order chunk partials [C][1][E] (no
// selection); returns C.
int launch_route_chunks_t1(const moe_layer_desc *d, const void *x, const void *w_router, float *partials,
                           void *stream, StageMarker *mk = nullptr);
// The one-token layer after the router's chunk partials, in two launches:
// selection fused with gate/up (h [k+S][d_ff] fp32), then down fused with
// the weighted combine into y.  idx/wt receive the routing.
bool t1_fused_applies(const moe_layer_desc *d, int32_t T);
// hmax: [k+S][d_ff/8] fp32 scratch.
void launch_t1_layer(const moe_layer_desc *d, const void *x, const moe_weights *w, const float *partials,
                     int n_chunks, int32_t *idx, float *wt, float *h, float *hmax, void *y, int32_t out_dtype,
                     void *stream, StageMarker *mk = nullptr);

// Dispatch: stable counting sort + prefix tables + the internal work plan.
// scratch holds dispatch_scratch_ints ints (per-workgroup counts for large N).
int64_t dispatch_scratch_ints(const moe_layer_desc *d, int32_t T);
// counts_ready: the per-segment counts in `scratch` were written by the
// router (route_counts_dispatch), so the counting pass is skipped.
void launch_dispatch(const moe_layer_desc *d, int32_t T, const int32_t *idx, int32_t tile_rows,
                     int32_t *order, int32_t *inv_order, int32_t *row_map, int32_t *expert_off,
                     int32_t *tile_off, int32_t *counters, PlanItem *act_items, PlanItem *tiles,
                     int32_t *scratch, void *stream, StageMarker *mk = nullptr, bool counts_ready = false);
// Slots per segment of the multi-workgroup dispatch (0 when T*k is small
// enough for one workgroup).
int64_t dispatch_segment_slots(const moe_layer_desc *d, int32_t T);
// The matrix-core router writes the multi-workgroup dispatch's counts.
bool route_counts_dispatch(const moe_layer_desc *d, int32_t T);

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
  uint16_t *xg = nullptr;  // group means of x16 (written by the expert FFN when the packed weights allow)
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
// the matrix-core path adds dg | du and the power-of-two exponents of its
// fp16 operands (per dg|du row and per dy row).
struct BwdScratch {
  float *gu;      // matrix cores: [R][2F] g | u per row; vector units: g [R][F] then u [R][F]
  float *v;       // [splits.v][R][F]
  float *dw;      // [R]
  float *dxr;     // [splits.dx][R][D]
  float *dgu;     // matrix-core path: [R][2F] fp32, dg then du
  int8_t *dgu_sh; // matrix-core path: [R] exponent of each dg|du row
  int8_t *dy_sh;  // matrix-core path: [T] exponent of each dy row
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
  size_t gu, v, dw, dxr, dgu, dgu_sh, dy_sh, wr_t, total;
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
