// moe_api.cpp -- the C ABI entry points: validate on the host, carve the
// caller's workspace, enqueue kernels on the caller's stream, never wait.
//
// One command stream per layer with no host wait between router and experts
// is the point of "MoE Optimization COMPLETE" ("Optimization Technique": the
// router result was read back on the CPU, costing a wait per layer); every
// entry point here only enqueues.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "moe_internal.h"

using namespace moe;

namespace moe {
KernelTimer *&kernel_timer() {
  static thread_local KernelTimer *t = nullptr;
  return t;
}
}  // namespace moe

namespace {

int hip_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

template <class T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

FfnScratch ffn_scratch(void *ws, const Workspace &L, bool x16_ready) {
  return FfnScratch{at<void>(ws, L.h), at<int8_t>(ws, L.hsh), at<void>(ws, L.x16), at<int8_t>(ws, L.xsh),
                    x16_ready, at<uint16_t>(ws, L.xg)};
}

int check_ws(const moe_layer_desc *d, int32_t T, const void *ws, size_t ws_bytes, Workspace *out) {
  *out = workspace_layout(d, T);
  if (validate_ptr(ws)) return MOE_E_INVALID;
  if (ws_bytes < out->total) return MOE_E_WORKSPACE;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_INVALID: return "MOE_E_INVALID: invalid descriptor, size, pointer or alignment";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: unsupported weight format";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace smaller than moe_workspace_size()";
    case MOE_E_HIP: return "MOE_E_HIP: HIP launch error";
    default: return "unknown moe_status";
  }
}

int moe_workspace_size(const moe_layer_desc *desc, int32_t T, size_t *bytes) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (!bytes) return MOE_E_INVALID;
  *bytes = workspace_layout(desc, T).total;
  return MOE_OK;
}

int moe_route(const moe_layer_desc *desc, int32_t T, const void *x, const void *w_router,
              const float *router_bias, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              void *stream) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if ((s = validate_ptr(x)) || (s = validate_ptr(w_router)) || (s = validate_ptr(router_bias, true)) ||
      (s = validate_ptr(topk_idx)) || (s = validate_ptr(topk_w)))
    return s;
  Workspace L;
  if ((s = check_ws(desc, T, ws, ws_bytes, &L))) return s;
  if (T == 0) return MOE_OK;
  launch_route(desc, T, x, w_router, router_bias, topk_idx, topk_w, at<float>(ws, L.route), nullptr, nullptr,
               nullptr, FusedDispatch{}, stream);
  return hip_status();
}

int moe_dispatch(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx, int32_t tile_rows,
                 int32_t *order, int32_t *inv_order, int32_t *row_map, int32_t *expert_off,
                 int32_t *tile_off, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (tile_rows < 1) return MOE_E_INVALID;
  if ((s = validate_ptr(topk_idx)) || (s = validate_ptr(order)) || (s = validate_ptr(inv_order)) ||
      (s = validate_ptr(row_map)) || (s = validate_ptr(expert_off)) || (s = validate_ptr(tile_off)))
    return s;
  Workspace L;
  if ((s = check_ws(desc, T, ws, ws_bytes, &L))) return s;
  if (T == 0) return MOE_OK;
  launch_dispatch(desc, T, topk_idx, tile_rows, order, inv_order, row_map, expert_off, tile_off,
                  at<int32_t>(ws, L.counters), at<PlanItem>(ws, L.act_items), at<PlanItem>(ws, L.tiles),
                  at<int32_t>(ws, L.dsp), stream);
  return hip_status();
}

int moe_expert_ffn(const moe_layer_desc *desc, int32_t T, const void *x, const int32_t *row_map,
                   const int32_t *expert_off, const moe_weights *w, float *y_sorted, void *ws,
                   size_t ws_bytes, void *stream) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if ((s = validate_ptr(x)) || (s = validate_ptr(row_map)) || (s = validate_ptr(expert_off)) ||
      (s = validate_ptr(y_sorted)))
    return s;
  if ((s = validate_weights(desc, w, false, true))) return s;
  Workspace L;
  if ((s = check_ws(desc, T, ws, ws_bytes, &L))) return s;
  if (T == 0) return MOE_OK;
  launch_plan(desc, T, expert_off, at<int32_t>(ws, L.counters), at<PlanItem>(ws, L.act_items),
              at<PlanItem>(ws, L.tiles), stream);
  launch_expert_ffn(desc, T, x, row_map, w, at<int32_t>(ws, L.counters), at<PlanItem>(ws, L.act_items),
                    at<PlanItem>(ws, L.tiles), L.max_tiles, ffn_scratch(ws, L, false), y_sorted, nullptr, stream);
  return hip_status();
}

int moe_combine(const moe_layer_desc *desc, int32_t T, const float *y_sorted, const int32_t *inv_order,
                const float *topk_w, void *y, int32_t out_dtype, void *stream) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16 && out_dtype != MOE_DT_F16) return MOE_E_INVALID;
  if ((s = validate_ptr(y_sorted)) || (s = validate_ptr(inv_order)) || (s = validate_ptr(topk_w)) ||
      (s = validate_ptr(y)))
    return s;
  if (T == 0) return MOE_OK;
  launch_combine(desc, T, y_sorted, nullptr, inv_order, topk_w, y, out_dtype, stream);
  return hip_status();
}

static int forward_impl(const moe_layer_desc *desc, int32_t T, const void *x, const moe_weights *w,
                        void *y, int32_t out_dtype, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                        size_t ws_bytes, void *stream, StageMarker *mk) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16 && out_dtype != MOE_DT_F16) return MOE_E_INVALID;
  if ((s = validate_ptr(x)) || (s = validate_ptr(y)) || (s = validate_ptr(topk_idx_out, true)) ||
      (s = validate_ptr(topk_w_out, true)))
    return s;
  if ((s = validate_weights(desc, w, true, true))) return s;
  Workspace L;
  if ((s = check_ws(desc, T, ws, ws_bytes, &L))) return s;
  if (T == 0) return MOE_OK;
  if (mk) mk->mark(nullptr);
  int32_t *idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.topk_idx);
  float *wt = topk_w_out ? topk_w_out : at<float>(ws, L.topk_w);
  if (t1_fused_applies(desc, T)) {
    // one token: router chunk partials, then selection + gate/up, then down +
    // combine (no dispatch: slot j of the token is its j-th expert)
    const int C = launch_route_chunks_t1(desc, x, w->w_router, at<float>(ws, L.route), stream, mk);
    launch_t1_layer(desc, x, w, at<float>(ws, L.route), C, idx, wt, at<float>(ws, L.h), at<float>(ws, L.y_sorted), y,
                    out_dtype, stream, mk);
    return hip_status();
  }
  const bool x16_ready = route_writes_x16(desc);
  const FusedDispatch dsp{at<int32_t>(ws, L.order), at<int32_t>(ws, L.inv_order), at<int32_t>(ws, L.row_map),
                          at<int32_t>(ws, L.expert_off), at<int32_t>(ws, L.tile_off), at<int32_t>(ws, L.counters),
                          at<PlanItem>(ws, L.act_items), at<PlanItem>(ws, L.tiles), 64,
                          plan_tile_rows(desc, T), desc->n_shared, at<int32_t>(ws, L.dsp)};
  launch_route(desc, T, x, w->w_router, w->router_bias, idx, wt, at<float>(ws, L.route), at<void>(ws, L.x16),
               at<int8_t>(ws, L.xsh), at<uint16_t>(ws, L.xg), dsp, stream, mk, w->w_router_packed);
  if (!route_fuses_dispatch(desc, T))
    launch_dispatch(desc, T, idx, 64, dsp.order, dsp.inv_order, dsp.row_map, dsp.expert_off, dsp.tile_off,
                    dsp.counters, dsp.act_items, dsp.tiles, at<int32_t>(ws, L.dsp), stream, mk,
                    route_counts_dispatch(desc, T));
  const int parts = ffn_down_parts(desc, T);
  int8_t *ys_sh = ys_f16e(desc, T) ? at<int8_t>(ws, L.ys_sh) : nullptr;
  launch_expert_ffn(desc, T, x, at<int32_t>(ws, L.row_map), w, at<int32_t>(ws, L.counters),
                    at<PlanItem>(ws, L.act_items), at<PlanItem>(ws, L.tiles), L.max_tiles,
                    ffn_scratch(ws, L, x16_ready), at<void>(ws, L.y_sorted), ys_sh, stream, mk, parts);
  launch_combine(desc, T, at<void>(ws, L.y_sorted), ys_sh, at<int32_t>(ws, L.inv_order), wt, y, out_dtype, stream,
                 mk, parts);
  return hip_status();
}

int moe_forward(const moe_layer_desc *desc, int32_t T, const void *x, const moe_weights *w, void *y,
                int32_t out_dtype, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                size_t ws_bytes, void *stream) {
  return forward_impl(desc, T, x, w, y, out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes, stream,
                      nullptr);
}

namespace {
// Hands each kernel of the call a (start, stop) event pair and names every
// kernel after the stage it belongs to.
struct EventMarker : StageMarker, KernelTimer {
  void *const *events;
  int32_t n_events, kernels = 0, named = 0;
  char *names;
  size_t names_len, pos = 0;
  bool next_events(hipEvent_t *start, hipEvent_t *stop) override {
    const int32_t k = kernels++;
    if (2 * k + 1 >= n_events) return false;
    *start = static_cast<hipEvent_t>(events[2 * k]);
    *stop = static_cast<hipEvent_t>(events[2 * k + 1]);
    return true;
  }
  void mark(const char *stage) override {
    for (; named < kernels; ++named) {
      if (!stage || !names || names_len == 0) continue;
      for (const char *p = (pos ? "," : ""); *p && pos + 1 < names_len; ++p) names[pos++] = *p;
      for (const char *p = stage; *p && pos + 1 < names_len; ++p) names[pos++] = *p;
      names[pos] = 0;
    }
  }
};

// Installs a kernel timer on this thread for one scope.
struct TimerScope {
  KernelTimer *saved;
  explicit TimerScope(KernelTimer *t) : saved(kernel_timer()) { kernel_timer() = t; }
  ~TimerScope() { kernel_timer() = saved; }
};
}  // namespace

int moe_forward_timed(const moe_layer_desc *desc, int32_t T, const void *x, const moe_weights *w,
                      void *y, int32_t out_dtype, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                      size_t ws_bytes, void *stream, void *const *events, int32_t n_events,
                      char *names, size_t names_len) {
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_E_INVALID;
  if (names && names_len) names[0] = 0;
  EventMarker mk;
  mk.events = events;
  mk.n_events = n_events;
  mk.names = names;
  mk.names_len = names_len;
  TimerScope scope(&mk);
  return forward_impl(desc, T, x, w, y, out_dtype, topk_idx_out, topk_w_out, ws, ws_bytes, stream, &mk);
}

int moe_router_packed_bytes(const moe_layer_desc *desc, size_t *bytes) {
  int s;
  if ((s = validate_desc(desc))) return s;
  if (!bytes) return MOE_E_INVALID;
  if (!router_pack_applies(desc)) return MOE_E_UNSUPPORTED;
  *bytes = router_packed_bytes(desc);
  return MOE_OK;
}

int moe_pack_router(const moe_layer_desc *desc, const void *w_router, void *out, void *stream) {
  size_t bytes = 0;
  int s;
  if ((s = moe_router_packed_bytes(desc, &bytes))) return s;
  if ((s = validate_ptr(w_router)) || (s = validate_ptr(out))) return s;
  launch_pack_router(desc, w_router, out, stream);
  return hip_status();
}

int moe_packed_bytes(const moe_layer_desc *desc, int32_t proj, size_t *bytes) {
  int s;
  if ((s = validate_desc(desc))) return s;
  if (!bytes) return MOE_E_INVALID;
  if (!affine(desc)) return MOE_E_UNSUPPORTED;
  PackedLayout L;
  if (!packed_layout(desc, proj, &L)) return MOE_E_INVALID;
  *bytes = L.total;
  return MOE_OK;
}

int moe_pack_weights(const moe_layer_desc *desc, int32_t proj, const void *w, const void *scales,
                     const void *biases, void *w_packed, void *stream) {
  size_t bytes = 0;
  int s;
  if ((s = moe_packed_bytes(desc, proj, &bytes))) return s;
  if ((s = validate_ptr(w)) || (s = validate_ptr(scales)) || (s = validate_ptr(biases)) ||
      (s = validate_ptr(w_packed)))
    return s;
  launch_pack(desc, proj, static_cast<const uint32_t *>(w), static_cast<const uint16_t *>(scales),
              static_cast<const uint16_t *>(biases), w_packed, stream);
  return hip_status();
}

int moe_backward_workspace_size(const moe_layer_desc *desc, int32_t T, size_t *bytes) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (!bytes) return MOE_E_INVALID;
  *bytes = backward_workspace_layout(desc, T).total;
  return MOE_OK;
}

int moe_backward(const moe_layer_desc *desc, int32_t T, const void *x, const moe_weights *w, const float *dy,
                 float *dx, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if ((s = validate_ptr(x)) || (s = validate_ptr(dy)) || (s = validate_ptr(dx))) return s;
  if ((s = validate_weights(desc, w, true, true))) return s;
  if (validate_ptr(ws)) return MOE_E_INVALID;
  const BwdWorkspace B = backward_workspace_layout(desc, T);
  if (ws_bytes < B.total) return MOE_E_WORKSPACE;
  if (T == 0) return MOE_OK;
  const Workspace &L = B.fwd;
  // the forward's routing and grouping, again (and the fp16 staging copy of x)
  int32_t *idx = at<int32_t>(ws, L.topk_idx);
  float *wt = at<float>(ws, L.topk_w);
  FusedDispatch counts_only{};
  counts_only.counts = at<int32_t>(ws, L.dsp);
  launch_route(desc, T, x, w->w_router, w->router_bias, idx, wt, at<float>(ws, L.route), at<void>(ws, L.x16),
               at<int8_t>(ws, L.xsh), nullptr, counts_only, stream, nullptr, w->w_router_packed);
  launch_dispatch(desc, T, idx, plan_tile_rows(desc, T), at<int32_t>(ws, L.order), at<int32_t>(ws, L.inv_order),
                  at<int32_t>(ws, L.row_map), at<int32_t>(ws, L.expert_off), at<int32_t>(ws, L.tile_off),
                  at<int32_t>(ws, L.counters), at<PlanItem>(ws, L.act_items), at<PlanItem>(ws, L.tiles),
                  at<int32_t>(ws, L.dsp), stream, nullptr, route_counts_dispatch(desc, T));
  const BwdScratch sc{at<float>(ws, B.gu),     at<float>(ws, B.v),       at<float>(ws, B.dw),
                      at<float>(ws, B.dxr),    at<float>(ws, B.dgu),     at<int8_t>(ws, B.dgu_sh),
                      at<int8_t>(ws, B.dy_sh), at<void>(ws, B.wr_t),     ffn_scratch(ws, L, route_writes_x16(desc))};
  launch_backward(desc, T, x, w, dy, idx, wt, at<int32_t>(ws, L.order), at<int32_t>(ws, L.inv_order),
                  at<int32_t>(ws, L.row_map), at<int32_t>(ws, L.counters), at<PlanItem>(ws, L.act_items),
                  at<PlanItem>(ws, L.tiles), L.max_tiles, sc, dx, stream);
  return hip_status();
}

}  // extern "C"
