// combine.hip -- score-weighted unsort of the expert outputs.
//
// y[t] = sum_j w[t][j] * y_sorted[inv_order[t*k + j]] + sum_s y_shared_s[t]:
// the weighted sum of "perf(moe): fused MoE expert decode kernel" ("What it
// does") gathered through inv_order as in DS4Server #112's _scatter_unsort.
// A gather per token instead of the PRD's atomic scatter-add keeps the fp32
// summation order fixed (slot order), so results are deterministic.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ys,
                                                      const int32_t *__restrict__ inv,
                                                      const float *__restrict__ w, int T, int K,
                                                      int S, int N, int D, void *__restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < D; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < K; ++j) {
      const int p = inv[int64_t(t) * K + j];
      if (unsigned(p) >= unsigned(N)) continue;
      const float wj = w[int64_t(t) * K + j];
      const float4 v = *reinterpret_cast<const float4 *>(ys + int64_t(p) * D + c);
      acc.x += wj * v.x;
      acc.y += wj * v.y;
      acc.z += wj * v.z;
      acc.w += wj * v.w;
    }
    for (int s = 0; s < S; ++s) {
      const float4 v = *reinterpret_cast<const float4 *>(ys + (int64_t(N) + int64_t(s) * T + t) * D + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if constexpr (OUT_BF16) {
      uint2 o;
      o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + int64_t(t) * D + c) = o;
    } else {
      *reinterpret_cast<float4 *>(static_cast<float *>(y) + int64_t(t) * D + c) = acc;
    }
  }
}

}  // namespace

void launch_combine(const moe_layer_desc *d, int32_t T, const float *y_sorted,
                    const int32_t *inv_order, const float *topk_w, void *y, int32_t out_dtype,
                    void *stream, StageMarker *mk) {
  const int N = T * d->top_k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out_dtype == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, y_sorted, inv_order, topk_w, T,
                       d->top_k, d->n_shared, N, d->d_model, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, y_sorted, inv_order, topk_w,
                       T, d->top_k, d->n_shared, N, d->d_model, y);
  if (mk) mk->mark("combine");
}

}  // namespace moe
