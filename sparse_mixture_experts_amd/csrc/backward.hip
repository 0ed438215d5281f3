// backward.hip -- the layer's backward pass with respect to x.
//
// "SwitchGLU: grouped-expert Metal kernels" (ml-explore/mlx-lm #2044),
// section "What": the grouped expert kernels carry a custom VJP so that
// training runs through the quantised experts.  With the weights fixed and the
// routing held at the forward's choice (the router and the dispatch run again
// here, so the routed rows and their grouping are those of the forward), for
// sorted row r (expert e, token t, slot weight c; shared rows c = 1):
//   g = Wg x_t, u = Wu x_t, h = glu(g, u)                         (kernel 1)
//   v = Wd^T dy_t                                                 (kernel 2)
//   dw_r = h . v (= dy_t . Wd h); dh = c v -> dg, du (GLU derivative)  (kernel 3)
//   dx_r = Wg^T dg + Wu^T du                                      (kernel 4)
//   dx_t = sum of its slots' dx_r in slot order + shared rows + W_r dl, with
//   dl the softmax backward of the slot weights from dw            (kernel 5)
// The forward's per-op rounding is not differentiated (the unrounded GLU).
// fp32 layers run kernels 1-4 here, all arithmetic fp32 on the vector units
// (each weight element is read where its row or column is reduced, for up to
// kMR routed rows at a time); 16-bit layers run the matrix-core versions of
// kernels 1-4 (backward_mfma.hip).  Kernel 5 serves both.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMR = 8;  // routed rows per pass

// One projection of every expert: N weight rows of K columns each (rows
// `row_off` .. of the stored [nre][K] matrix of an expert).
struct WView {
  const void *w;
  const uint16_t *sc, *bi;
  int N, K, row_off, nre;
};
struct WFormat {
  int act_dtype;  // moe_dtype of dense weights and of scales/biases
  int bits;       // 0: dense; 4 or 8: affine codes
  int group;
};

// Weight (row n, column k) of expert e as fp32.
__device__ __forceinline__ float wload(const WFormat &f, const WView &v, int e, int n, int k) {
  const int64_t row = int64_t(e) * v.nre + v.row_off + n;
  if (f.bits == 0) {
    const int64_t i = row * v.K + k;
    if (f.act_dtype == MOE_DT_F32) return static_cast<const float *>(v.w)[i];
    const uint32_t h = static_cast<const uint16_t *>(v.w)[i];
    return f.act_dtype == MOE_DT_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
  }
  const int per = 32 / f.bits;
  const uint32_t word = static_cast<const uint32_t *>(v.w)[row * (v.K / per) + k / per];
  const uint32_t q = (word >> (f.bits * (k % per))) & ((1u << f.bits) - 1u);
  const int64_t si = (int64_t(e) * (v.K / f.group) + k / f.group) * v.nre + v.row_off + n;
  const uint32_t sh = v.sc[si], bh = v.bi[si];
  const float s = f.act_dtype == MOE_DT_F16 ? f16_bits_to_f32(sh) : bf16_bits_to_f32(sh);
  const float b = f.act_dtype == MOE_DT_F16 ? f16_bits_to_f32(bh) : bf16_bits_to_f32(bh);
  return __builtin_fmaf(s, float(q), b);
}

__device__ __forceinline__ float act_load(int dt, const void *p, int64_t i) {
  if (dt == MOE_DT_F32) return static_cast<const float *>(p)[i];
  const uint32_t h = static_cast<const uint16_t *>(p)[i];
  return dt == MOE_DT_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}

struct BwdArgs {
  WFormat fmt;
  WView gate, up, down;
  const void *x;
  const float *dy;
  const int32_t *row_map, *order, *inv_order;
  const float *topk_w;
  const int32_t *counters;
  const PlanItem *items;
  int T, N, K, D, F, E, S, geglu, renorm;
  const void *w_router;   // [D][E]
  const void *wr_t;       // [E][D] (the router matrix transposed)
  const float *router_bias;
  float *g, *u, *v, *dw, *dxr;
  int dx_splits;          // partial sums of the rows' dx, [dx_splits][R][D]
  float *dx;
  const int32_t *topk_idx;
};

// Token of sorted row r (routed rows through row_map, shared rows by position).
__device__ __forceinline__ int token_of(const BwdArgs &a, int r) {
  return r < a.N ? a.row_map[r] : (r - a.N) % a.T;
}

// 1. g, u for the rows of one plan item.  Block (fb, item): 4 waves x 4
// columns f each; the lanes split the reduction over d (lane l takes d = l,
// l + 64, ...) and a wave sum finishes each dot product.
__global__ __launch_bounds__(kThreads) void bwd_gate_up_kernel(BwdArgs a) {
  if (int(blockIdx.y) >= a.counters[0]) return;
  const PlanItem it = a.items[blockIdx.y];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  for (int q = 0; q < 4; ++q) {
    const int f = blockIdx.x * 16 + wave * 4 + q;
    if (f >= a.F) break;  // uniform per wave
    for (int r0 = 0; r0 < it.rows; r0 += kMR) {
      const int mr = min(kMR, it.rows - r0);
      float ag[kMR], au[kMR];
      int tok[kMR];
#pragma unroll
      for (int m = 0; m < kMR; ++m) {
        ag[m] = au[m] = 0.f;
        tok[m] = m < mr ? token_of(a, it.row0 + r0 + m) : 0;
      }
      for (int k = lane; k < a.D; k += kWave) {
        const float wg = wload(a.fmt, a.gate, it.expert, f, k), wu = wload(a.fmt, a.up, it.expert, f, k);
#pragma unroll
        for (int m = 0; m < kMR; ++m) {
          if (m < mr) {
            const float xv = act_load(a.fmt.act_dtype, a.x, int64_t(tok[m]) * a.D + k);
            ag[m] = __builtin_fmaf(xv, wg, ag[m]);
            au[m] = __builtin_fmaf(xv, wu, au[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kMR; ++m) {
        if (m < mr) {
          const float gs = wave_sum(ag[m]), us = wave_sum(au[m]);
          if (lane == 0) {
            const int64_t o = int64_t(it.row0 + r0 + m) * a.F + f;
            a.g[o] = gs;
            a.u[o] = us;
          }
        }
      }
    }
  }
}

// 2. v = Wd^T dy for the rows of one plan item.  Block (cb, item): thread =
// column f of the down matrix, the loop runs over its rows m (consecutive
// threads read consecutive elements of a row).
__global__ __launch_bounds__(kThreads) void bwd_down_t_kernel(BwdArgs a) {
  if (int(blockIdx.y) >= a.counters[0]) return;
  const PlanItem it = a.items[blockIdx.y];
  const int f = blockIdx.x * kThreads + threadIdx.x;
  const int fc = min(f, a.F - 1);
  for (int r0 = 0; r0 < it.rows; r0 += kMR) {
    const int mr = min(kMR, it.rows - r0);
    float acc[kMR];
    int tok[kMR];
#pragma unroll
    for (int m = 0; m < kMR; ++m) {
      acc[m] = 0.f;
      tok[m] = m < mr ? token_of(a, it.row0 + r0 + m) : 0;
    }
    for (int d = 0; d < a.D; ++d) {
      const float w = wload(a.fmt, a.down, it.expert, d, fc);
#pragma unroll
      for (int m = 0; m < kMR; ++m)
        if (m < mr) acc[m] = __builtin_fmaf(a.dy[int64_t(tok[m]) * a.D + d], w, acc[m]);
    }
    if (f < a.F) {
#pragma unroll
      for (int m = 0; m < kMR; ++m)
        if (m < mr) a.v[int64_t(it.row0 + r0 + m) * a.F + f] = acc[m];
    }
  }
}

// 3. Per sorted row: dw = h . v, and dg, du in place of g, u.
__global__ __launch_bounds__(kThreads) void bwd_glu_kernel(BwdArgs a) {
  __shared__ float part[kThreads];
  const int r = blockIdx.x;
  const float c = r < a.N ? a.topk_w[a.order[r]] : 1.0f;
  float dwp = 0.f;
  for (int f = threadIdx.x; f < a.F; f += kThreads) {
    const int64_t o = int64_t(r) * a.F + f;
    const float g = a.g[o], u = a.u[o], v = a.v[o];
    float act, dact;  // the gate's activation and its derivative
    gate_act_grad(g, a.geglu != 0, act, dact);
    dwp = __builtin_fmaf(act * u, v, dwp);
    const float dh = c * v;
    a.g[o] = dh * u * dact;
    a.u[o] = dh * act;
  }
  part[threadIdx.x] = dwp;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dw[r] = part[0];
}

// 4. dx_r = Wg^T dg + Wu^T du for the rows of one plan item.  Block (cb,
// item): thread = column k of the gate/up matrices, the loop runs over f.
__global__ __launch_bounds__(kThreads) void bwd_gate_up_t_kernel(BwdArgs a) {
  if (int(blockIdx.y) >= a.counters[0]) return;
  const PlanItem it = a.items[blockIdx.y];
  const int k = blockIdx.x * kThreads + threadIdx.x;
  const int kc = min(k, a.D - 1);
  for (int r0 = 0; r0 < it.rows; r0 += kMR) {
    const int mr = min(kMR, it.rows - r0);
    float acc[kMR];
#pragma unroll
    for (int m = 0; m < kMR; ++m) acc[m] = 0.f;
    for (int f = 0; f < a.F; ++f) {
      const float wg = wload(a.fmt, a.gate, it.expert, f, kc), wu = wload(a.fmt, a.up, it.expert, f, kc);
#pragma unroll
      for (int m = 0; m < kMR; ++m) {
        if (m < mr) {
          const int64_t o = int64_t(it.row0 + r0 + m) * a.F + f;
          acc[m] = __builtin_fmaf(a.g[o], wg, acc[m]);
          acc[m] = __builtin_fmaf(a.u[o], wu, acc[m]);
        }
      }
    }
    if (k < a.D) {
#pragma unroll
      for (int m = 0; m < kMR; ++m)
        if (m < mr) a.dxr[int64_t(it.row0 + r0 + m) * a.D + k] = acc[m];
    }
  }
}

// Four consecutive elements of a layer-dtype array as fp32.
template <int DT>
__device__ __forceinline__ float4 load4(const void *p, int64_t i) {
  if constexpr (DT == kDtF32) return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
  const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
  return make_float4(half_lo<DT>(u.x), half_hi<DT>(u.x), half_lo<DT>(u.y), half_hi<DT>(u.y));
}
__device__ __forceinline__ void add4(float4 &a, const float4 &b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

// 5. Per token: router gradient and the sum over its rows.  With
// renormalisation the slot weights are the softmax of the selected logits,
// dl_j = w_j (dw_j - sum_i w_i dw_i); without it they are the softmax over all
// E logits (recomputed here, fp32, ascending d), dl_e = p_e (dw(e) - sum_j
// w_j dw_j).  dx_t = its slots' rows (slot order) + shared rows + W_r dl, four
// columns per thread and step.  DT: the layer's dtype (kDt*).
template <int DT>
__global__ __launch_bounds__(kThreads) void bwd_token_kernel(BwdArgs a) {
  __shared__ float dl[kMaxExperts];  // renormalised: per slot; else per expert
  __shared__ float red[kThreads];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t s0 = int64_t(t) * a.K;
  float dot = 0.f;
  for (int j = 0; j < a.K; ++j) dot += a.topk_w[s0 + j] * a.dw[a.inv_order[s0 + j]];
  if (a.renorm) {
    if (tid < a.K) dl[tid] = a.topk_w[s0 + tid] * (a.dw[a.inv_order[s0 + tid]] - dot);
  } else {
    for (int e = tid; e < a.E; e += kThreads) {
      float l = 0.f;
      for (int d = 0; d < a.D; ++d)
        l = __builtin_fmaf(load_act<DT>(a.x, int64_t(t) * a.D + d), load_act<DT>(a.w_router, int64_t(d) * a.E + e), l);
      dl[e] = a.router_bias ? l + a.router_bias[e] : l;
    }
    float mx = -INFINITY;
    for (int e = tid; e < a.E; e += kThreads) mx = fmaxf(mx, dl[e]);
    red[tid] = mx;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
      __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float z = 0.f;
    for (int e = tid; e < a.E; e += kThreads) z += expf(dl[e] - mx);
    red[tid] = z;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    z = red[0];
    for (int e = tid; e < a.E; e += kThreads) dl[e] = -(expf(dl[e] - mx) / z) * dot;
    __syncthreads();
    if (tid == 0)
      for (int j = 0; j < a.K; ++j) dl[a.topk_idx[s0 + j]] += a.topk_w[s0 + j] * a.dw[a.inv_order[s0 + j]];
  }
  __syncthreads();
  const int64_t R = int64_t(a.N) + int64_t(a.S) * a.T, split = R * a.D;
  for (int k = 4 * tid; k < a.D; k += 4 * kThreads) {
    auto row_dx = [&](int64_t r) {  // one row's dx: its split partials in split order
      const float *p = a.dxr + r * a.D + k;
      float4 v = *reinterpret_cast<const float4 *>(p);
      for (int z = 1; z < a.dx_splits; ++z) add4(v, *reinterpret_cast<const float4 *>(p + z * split));
      return v;
    };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int j = 0; j < a.K; ++j) add4(acc, row_dx(a.inv_order[s0 + j]));
    for (int s = 0; s < a.S; ++s) add4(acc, row_dx(int64_t(a.N) + int64_t(s) * a.T + t));
    float4 rg = make_float4(0.f, 0.f, 0.f, 0.f);
    auto router_row = [&](int e, float c) {  // rg += c * (row e of W_r^T)
      const float4 w = load4<DT>(a.wr_t, int64_t(e) * a.D + k);
      rg.x = __builtin_fmaf(w.x, c, rg.x);
      rg.y = __builtin_fmaf(w.y, c, rg.y);
      rg.z = __builtin_fmaf(w.z, c, rg.z);
      rg.w = __builtin_fmaf(w.w, c, rg.w);
    };
    if (a.renorm) {
#pragma unroll 4
      for (int j = 0; j < a.K; ++j) router_row(a.topk_idx[s0 + j], dl[j]);
    } else {
      for (int e = 0; e < a.E; ++e) router_row(e, dl[e]);
    }
    add4(acc, rg);
    *reinterpret_cast<float4 *>(a.dx + int64_t(t) * a.D + k) = acc;
  }
}

// The router matrix [D][E] transposed to [E][D] through 32x32 LDS tiles
// (ESZ-byte elements), so that the per-token kernel reads its rows whole.
template <typename Elt>
__global__ __launch_bounds__(256) void transpose_kernel(const Elt *src, int rows, int cols, Elt *dst) {
  __shared__ Elt tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  for (int i = ty; i < 32; i += 8)
    if (r0 + i < rows && c0 + tx < cols) tile[i][tx] = src[int64_t(r0 + i) * cols + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 32; i += 8)
    if (c0 + i < cols && r0 + tx < rows) dst[int64_t(c0 + i) * rows + r0 + tx] = tile[tx][i];
}

}  // namespace

void launch_backward(const moe_layer_desc *d, int32_t T, const void *x, const moe_weights *w, const float *dy,
                     const int32_t *topk_idx, const float *topk_w, const int32_t *order, const int32_t *inv_order,
                     const int32_t *row_map, const int32_t *counters, const PlanItem *items, const PlanItem *tiles,
                     int64_t max_tiles, const BwdScratch &sc, float *dx, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_model, F = d->d_ff, E = d->n_experts, S = d->n_shared, K = d->top_k;
  const int N = T * K, R = N + S * T;
  const int max_items = std::min(E, N) + S;
  const bool fused = d->gate_up_fused;
  const int bits = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : d->w_format == MOE_WF_AFFINE_Q4 ? 4 : 0;
  const moe_proj &pg = fused ? w->gate_up : w->gate, &pu = fused ? w->gate_up : w->up;
  auto view = [&](const moe_proj &p, int n, int k, int row_off, int nre) {
    return WView{p.w, static_cast<const uint16_t *>(p.scales), static_cast<const uint16_t *>(p.biases), n, k,
                 row_off, nre};
  };
  const BwdSplits sp = backward_splits(d, T);
  BwdArgs a{WFormat{d->act_dtype, bits, d->group_size},
            view(pg, F, D, 0, fused ? 2 * F : F), view(pu, F, D, fused ? F : 0, fused ? 2 * F : F),
            view(w->down, D, F, 0, D), x, dy, row_map, order, inv_order, topk_w, counters, items,
            T, N, K, D, F, E, S, d->activation == MOE_ACT_GEGLU, d->renormalize, w->w_router, sc.wr_t,
            w->router_bias, sc.gu, sc.gu + int64_t(R) * F, sc.v, sc.dw, sc.dxr, sp.dx, dx, topk_idx};
  const dim3 tgrid((E + 31) / 32, (D + 31) / 32);
  if (d->act_dtype == MOE_DT_F32)
    hipLaunchKernelGGL(transpose_kernel<float>, tgrid, dim3(256), 0, s, static_cast<const float *>(w->w_router), D,
                       E, static_cast<float *>(sc.wr_t));
  else
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, tgrid, dim3(256), 0, s,
                       static_cast<const uint16_t *>(w->w_router), D, E, static_cast<uint16_t *>(sc.wr_t));
  if (use_mfma(d)) {
    launch_backward_mfma(d, T, x, w, dy, topk_w, order, row_map, counters, tiles, max_tiles, sc, stream);
  } else {
    hipLaunchKernelGGL(bwd_gate_up_kernel, dim3((F + 15) / 16, max_items), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_down_t_kernel, dim3((F + kThreads - 1) / kThreads, max_items), dim3(kThreads), 0, s,
                       a);
    hipLaunchKernelGGL(bwd_glu_kernel, dim3(R), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_gate_up_t_kernel, dim3((D + kThreads - 1) / kThreads, max_items), dim3(kThreads), 0,
                       s, a);
  }
  if (d->act_dtype == MOE_DT_F32) hipLaunchKernelGGL(bwd_token_kernel<kDtF32>, dim3(T), dim3(kThreads), 0, s, a);
  else if (d->act_dtype == MOE_DT_F16) hipLaunchKernelGGL(bwd_token_kernel<kDtF16>, dim3(T), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(bwd_token_kernel<kDtBF16>, dim3(T), dim3(kThreads), 0, s, a);
}

}  // namespace moe
