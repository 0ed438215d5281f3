// moe_validate.cpp -- host-side argument checks and workspace layout.
// No HIP calls here: everything in this file runs before anything is enqueued,
// so an invalid call returns an error with no device work and no side effects.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

static bool is_bool(int32_t v) { return v == 0 || v == 1; }

int validate_desc(const moe_layer_desc *d) {
  if (!d) return MOE_E_INVALID;
  if (d->act_dtype != MOE_DT_F32 && d->act_dtype != MOE_DT_BF16 && d->act_dtype != MOE_DT_F16)
    return MOE_E_INVALID;
  if (d->w_format != MOE_WF_DENSE && !affine(d)) return MOE_E_INVALID;
  if (!is_bool(d->gate_up_fused) || !is_bool(d->glu_round) || !is_bool(d->renormalize))
    return MOE_E_INVALID;
  if (d->activation != MOE_ACT_SWIGLU && d->activation != MOE_ACT_GEGLU) return MOE_E_INVALID;
  if (d->d_model <= 0 || d->d_ff <= 0 || d->d_model > 16384 || d->d_ff > 16384) return MOE_E_INVALID;
  if (d->n_experts < 1 || d->n_experts > kMaxExperts) return MOE_E_INVALID;
  if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->n_experts) return MOE_E_INVALID;
  if (d->n_shared < 0 || d->n_shared > kMaxShared) return MOE_E_INVALID;
  if (d->glu_round && d->act_dtype == MOE_DT_F32) return MOE_E_INVALID;  // rounds to a 16-bit dtype
  if (affine(d)) {
    // The affine formats carry scales/biases in the 16-bit activation dtype;
    // groups of 32, 64 or 128 along both reduction dims, which the matrix-core
    // kernels walk in steps of 64.
    if (d->act_dtype == MOE_DT_F32) return MOE_E_UNSUPPORTED;
    const int g = d->group_size;
    if (g != 32 && g != 64 && g != 128) return MOE_E_UNSUPPORTED;
    if (d->d_model % 64 || d->d_ff % 64 || d->d_model % g || d->d_ff % g) return MOE_E_INVALID;
  } else {
    if (d->d_model % 8 || d->d_ff % 8) return MOE_E_INVALID;
  }
  return MOE_OK;
}

int validate_T(int32_t T) {
  // T*k and the shared rows must stay far below 2^31 sorted rows.
  if (T < 0 || T > (1 << 20)) return MOE_E_INVALID;
  return MOE_OK;
}

int validate_ptr(const void *p, bool may_be_null) {
  if (!p) return may_be_null ? MOE_OK : MOE_E_INVALID;
  if (reinterpret_cast<uintptr_t>(p) % 16) return MOE_E_INVALID;
  return MOE_OK;
}

static int validate_proj(const moe_layer_desc *d, const moe_proj &p) {
  int s = validate_ptr(p.w);
  if (s) return s;
  if (affine(d)) {
    if ((s = validate_ptr(p.scales))) return s;
    if ((s = validate_ptr(p.biases))) return s;
    if ((s = validate_ptr(p.w_packed, true))) return s;
  } else if (p.w_packed) {
    return MOE_E_INVALID;  // the packed copy exists for affine codes only
  }
  return MOE_OK;
}

// Rows N and reduction K of projection `proj` (moe_projection); false when
// the descriptor does not use it.
bool proj_shape(const moe_layer_desc *d, int32_t proj, int *N, int *K) {
  switch (proj) {
    case MOE_PROJ_GATE:
    case MOE_PROJ_UP:
      if (d->gate_up_fused) return false;
      *N = d->d_ff, *K = d->d_model;
      return true;
    case MOE_PROJ_GATE_UP:
      if (!d->gate_up_fused) return false;
      *N = 2 * d->d_ff, *K = d->d_model;
      return true;
    case MOE_PROJ_DOWN:
      *N = d->d_model, *K = d->d_ff;
      return true;
    default:
      return false;
  }
}

static size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

bool packed_layout(const moe_layer_desc *d, int32_t proj, PackedLayout *out) {
  PackedLayout L{};
  if (!affine(d) || !proj_shape(d, proj, &L.N, &L.K)) return false;
  const int b = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : 4;
  const int64_t M = int64_t(d->n_experts) + d->n_shared;
  L.nslab = (L.K + 127) / 128;
  L.SW = 128 * b / 32;
  L.GPS = 128 / d->group_size;
  L.G = L.K / d->group_size;
  L.GP = (L.G + 31) / 32 * 32;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.codes = take(size_t(M) * L.N * L.nslab * L.SW * 4);
  L.scales = take(size_t(M) * L.N * L.nslab * L.GPS * 2);
  L.biases = take(size_t(M) * L.N * L.GP * 2);
  L.flags = take(size_t(M) * 4);
  L.total = o;
  *out = L;
  return true;
}

int xg_groups_padded(const moe_layer_desc *d) {
  const int G = d->d_model / d->group_size;
  return (G + 31) / 32 * 32;
}

XgOut xg_out(const moe_layer_desc *d, uint16_t *xg) {
  if (!xg || !affine(d) || !use_mfma(d)) return XgOut{nullptr, 0, 0};
  return XgOut{xg, d->group_size, xg_groups_padded(d)};
}

int validate_weights(const moe_layer_desc *d, const moe_weights *w, bool need_router,
                     bool need_experts) {
  if (!w) return MOE_E_INVALID;
  int s;
  if (need_router) {
    if ((s = validate_ptr(w->w_router))) return s;
    if ((s = validate_ptr(w->router_bias, true))) return s;
    if ((s = validate_ptr(w->w_router_packed, true))) return s;
    // a prepared router only where the matrix-core router can use one
    if (w->w_router_packed && !router_pack_applies(d)) return MOE_E_INVALID;
  }
  if (need_experts) {
    if (d->gate_up_fused) {
      if ((s = validate_proj(d, w->gate_up))) return s;
    } else {
      if ((s = validate_proj(d, w->gate))) return s;
      if ((s = validate_proj(d, w->up))) return s;
    }
    if ((s = validate_proj(d, w->down))) return s;
  }
  return MOE_OK;
}

Workspace workspace_layout(const moe_layer_desc *d, int32_t T) {
  Workspace ws{};
  const int64_t N = int64_t(T) * d->top_k;
  const int64_t S = d->n_shared, E = d->n_experts;
  const int64_t rows = N + S * T;
  const int64_t tiles_per_shared = (T + kMinTileRows - 1) / kMinTileRows;
  ws.max_tiles = (N + kMinTileRows - 1) / kMinTileRows + std::min<int64_t>(E, N) + S * tiles_per_shared + 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  ws.topk_idx = take(size_t(N) * 4);
  ws.topk_w = take(size_t(N) * 4);
  ws.route = take(size_t(route_scratch_floats(d, T)) * 4);
  ws.order = take(size_t(N) * 4);
  ws.inv_order = take(size_t(N) * 4);
  ws.row_map = take(size_t(N) * 4);
  ws.expert_off = take(size_t(E + 1) * 4);
  ws.tile_off = take(size_t(E + 1) * 4);
  ws.counters = take(64 * 4);
  ws.dsp = take(size_t(dispatch_scratch_ints(d, T)) * 4);
  ws.act_items = take(size_t(E + S) * sizeof(PlanItem));
  ws.tiles = take(size_t(ws.max_tiles) * sizeof(PlanItem));
  // h rows; the one-token layer keeps them as fp32 ([k+S][d_ff]), which the
  // 16-bit rows of two tokens already cover, so the size stays non-decreasing in T
  const int64_t h_one_token = T >= 1 ? (int64_t(d->top_k) + S) * d->d_ff * 4 : 0;
  ws.h = take(size_t(std::max<int64_t>(rows * d->d_ff * h_bytes(d), h_one_token)));
  const bool q4 = affine(d);
  ws.hsh = take(q4 ? size_t(rows) * ((d->d_ff + kHBlock - 1) / kHBlock) : 0);
  ws.x16 = take(q4 ? size_t(T) * d->d_model * 2 : 0);
  ws.xsh = take(q4 ? size_t(T) : 0);
  ws.xg = take(q4 && use_mfma(d) ? size_t(T) * xg_groups_padded(d) * 2 : 0);
  ws.y_sorted = take(size_t(ys_workspace_bytes(d, T)));
  ws.ys_sh = take(use_mfma(d) ? size_t(rows) * (d->d_model / kYsBlock) : 0);
  ws.total = o;
  return ws;
}

BwdWorkspace backward_workspace_layout(const moe_layer_desc *d, int32_t T) {
  BwdWorkspace b{};
  b.fwd = workspace_layout(d, T);
  const int64_t rows = int64_t(T) * d->top_k + int64_t(d->n_shared) * T;
  const BwdSplits sp = backward_splits(d, T);
  const bool mc = use_mfma(d);
  size_t o = b.fwd.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  b.gu = take(size_t(rows) * 2 * d->d_ff * 4);
  b.v = take(size_t(sp.v) * rows * d->d_ff * 4);
  b.dw = take(size_t(rows) * 4);
  b.dxr = take(size_t(sp.dx) * rows * d->d_model * 4);
  b.dgu = take(mc ? size_t(rows) * 2 * d->d_ff * 4 : 0);
  b.dgu_sh = take(mc ? size_t(rows) : 0);
  b.dy_sh = take(mc ? size_t(T) : 0);
  b.wr_t = take(size_t(d->n_experts) * d->d_model * act_bytes(d));
  b.total = o;
  return b;
}

}  // namespace moe
