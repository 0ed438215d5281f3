// route.hip -- router: logits, softmax and top-k, all on the device.
//
// The pages move router matmul, softmax and top-K selection onto the GPU so
// that no host wait sits between router and experts ("MoE Optimization
// COMPLETE", sections "Optimization Technique" and "Mega Kernel
// Architecture"; PRD "5.5 real sparse MoE kernels (Metal)", "Scope - in":
// top-K routing kernel with no host roundtrip).
//
// Logit arithmetic is fixed so that expert indices are reproducible bit for
// bit: for each (token, expert) the reduction over d runs in chunks of 64
// consecutive columns; a chunk is a sequential fma chain starting at +0, the
// chunk partials are added in ascending order to an accumulator starting at
// +0, and the bias is added last.  Each lane owns one expert and TT tokens,
// so the fma chains of one lane are independent and keep the VALU busy; the
// router column reads are coalesced across lanes (W_router is [d][E]).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TT = 8;      // tokens per workgroup
constexpr int SLAB = 512;  // columns of x staged in LDS at a time (multiple of 64)

// (v, e) ranks before (bv, be): larger logit first, ties to the lower index.
__device__ __forceinline__ bool ranks_before(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

template <bool BF16>
__global__ __launch_bounds__(256) void route_kernel(const void *__restrict__ x,
                                                    const void *__restrict__ wr,
                                                    const float *__restrict__ bias, int T, int D,
                                                    int E, int K, int renorm,
                                                    int32_t *__restrict__ idx_out,
                                                    float *__restrict__ w_out) {
  __shared__ float xs[SLAB][TT];
  extern __shared__ float logits[];  // [TT][E]

  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, T - t0);
  const int tid = threadIdx.x;

  for (int eg = 0; eg < E; eg += blockDim.x) {
    const int e = eg + tid;
    const bool active = e < E;
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
    for (int s0 = 0; s0 < D; s0 += SLAB) {
      const int s1 = min(s0 + SLAB, D);
      __syncthreads();
      for (int q = tid; q < TT * SLAB; q += blockDim.x) {
        const int t = q / SLAB, c = q % SLAB;
        float v = 0.0f;
        if (t < nt && s0 + c < s1) v = load_act<BF16>(x, int64_t(t0 + t) * D + s0 + c);
        xs[c][t] = v;
      }
      __syncthreads();
      if (active) {
        for (int c0 = s0; c0 < s1; c0 += 64) {
          const int c1 = min(c0 + 64, s1);
          float p[TT];
#pragma unroll
          for (int t = 0; t < TT; ++t) p[t] = 0.0f;
          for (int i = c0; i < c1; ++i) {
            const float w = load_act<BF16>(wr, int64_t(i) * E + e);
#pragma unroll
            for (int t = 0; t < TT; ++t) p[t] = __builtin_fmaf(xs[i - s0][t], w, p[t]);
          }
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[t] = acc[t] + p[t];
        }
      }
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < TT; ++t) logits[t * E + e] = bias ? acc[t] + bias[e] : acc[t];
    }
  }
  __syncthreads();

  // Selection and weights: one wave per token.  After each butterfly argmax
  // every lane holds the same winner, so lane j keeps the winner of round j.
  const int wave = tid / kWave, lane = lane_id(), nwaves = blockDim.x / kWave;
  for (int t = wave; t < nt; t += nwaves) {
    const float *l = logits + t * E;
    uint32_t taken = 0;  // bit m: expert lane + 64*m already selected
    int my_e = 0;
    float my_l = 0.0f, top = 0.0f;
    for (int j = 0; j < K; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
      for (int m = 0, e = lane; e < E; ++m, e += kWave) {
        if ((taken >> m) & 1u) continue;
        const float v = l[e];
        if (ranks_before(v, e, bv, be)) { bv = v; be = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ranks_before(ov, oe, bv, be)) { bv = ov; be = oe; }
      }
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
      if (j == 0) top = bv;
      if (lane == j) { my_e = be; my_l = bv; }
    }
    // fp32 softmax over all E logits (the top-1 logit is the maximum).
    float z = 0.0f;
    for (int e = lane; e < E; e += kWave) z += expf(l[e] - top);
    z = wave_sum(z);
    const float p = expf(my_l - top) / z;
    float w = p;
    if (renorm) {
      float psum = 0.0f;
      for (int j = 0; j < K; ++j) psum = psum + __shfl(p, j, kWave);
      w = p / psum;
    }
    if (lane < K) {
      idx_out[int64_t(t0 + t) * K + lane] = my_e;
      w_out[int64_t(t0 + t) * K + lane] = w;
    }
  }
}

}  // namespace

void launch_route(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router,
                  const float *bias, int32_t *idx, float *w, void *stream, StageMarker *mk) {
  const int E = d->n_experts;
  const int threads = E >= 256 ? 256 : ((E + kWave - 1) / kWave) * kWave;
  const dim3 grid((T + TT - 1) / TT);
  const size_t lds = size_t(TT) * E * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->act_dtype == MOE_DT_BF16)
    hipLaunchKernelGGL(route_kernel<true>, grid, dim3(threads), lds, s, x, w_router, bias, T,
                       d->d_model, E, d->top_k, d->renormalize, idx, w);
  else
    hipLaunchKernelGGL(route_kernel<false>, grid, dim3(threads), lds, s, x, w_router, bias, T,
                       d->d_model, E, d->top_k, d->renormalize, idx, w);
  if (mk) mk->mark("route");
}

}  // namespace moe
