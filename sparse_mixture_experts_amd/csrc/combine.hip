// combine.hip -- score-weighted unsort of the expert outputs.
//
// y[t] = sum_j w[t][j] * y_sorted[inv_order[t*k + j]] + sum_s y_shared_s[t]:
// the weighted sum of "perf(moe): fused MoE expert decode kernel" ("What it
// does") gathered through inv_order as in DS4Server #112's _scatter_unsort.
// A gather per token instead of the PRD's atomic scatter-add keeps the fp32
// summation order fixed (slot order), so results are deterministic.
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 8;  // columns per thread (one 16-byte bf16 load, two fp32 ones)

// Eight consecutive expert-output values, as loaded (bf16: one 16-byte load;
// fp32: two) and as fp32.
template <bool YS_BF16>
struct Row8 {
  uint4 u[YS_BF16 ? 1 : 2];
};
template <bool YS_BF16>
__device__ __forceinline__ Row8<YS_BF16> load8(const void *ys, int64_t i) {
  Row8<YS_BF16> r;
  if constexpr (YS_BF16) {
    r.u[0] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(ys) + i);
  } else {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const float *>(ys) + i);
    r.u[0] = q[0];
    r.u[1] = q[1];
  }
  return r;
}
template <bool YS_BF16>
__device__ __forceinline__ void widen8(const Row8<YS_BF16> &r, float v[8]) {
  if constexpr (YS_BF16) {
    const uint4 u = r.u[0];
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v[4 * h] = __uint_as_float(r.u[h].x); v[4 * h + 1] = __uint_as_float(r.u[h].y);
      v[4 * h + 2] = __uint_as_float(r.u[h].z); v[4 * h + 3] = __uint_as_float(r.u[h].w);
    }
  }
}

// Block (t, cb): token t, columns cb*256*8 ..; each thread 8 columns.  The
// token's slot positions and weights are uniform (scalar loads); then all
// slot rows of a thread (up to 16 bf16 or 8 fp32 rows per round) are in
// flight together before they are summed in slot order.
template <bool YS_BF16, int OUT_DT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void *__restrict__ ys,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ w, int T, int K, int S,
                                                           int N, int D, void *__restrict__ y) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * kCols;
  if (c >= D) return;
  float acc[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
  constexpr int kSlots = YS_BF16 ? 16 : 8;
  for (int j0 = 0; j0 < K; j0 += kSlots) {
    Row8<YS_BF16> r[kSlots];
    float wj[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int j = min(j0 + u, K - 1);
      const int p = inv[int64_t(t) * K + j];
      const bool ok = j0 + u < K && unsigned(p) < unsigned(N);
      wj[u] = ok ? w[int64_t(t) * K + j] : 0.f;
      r[u] = load8<YS_BF16>(ys, int64_t(ok ? p : 0) * D + c);
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
      if (j0 + u < K) {
        float v[kCols];
        widen8<YS_BF16>(r[u], v);
#pragma unroll
        for (int i = 0; i < kCols; ++i) acc[i] += wj[u] * v[i];
      }
  }
  for (int s = 0; s < S; ++s) {
    float v[kCols];
    widen8<YS_BF16>(load8<YS_BF16>(ys, (int64_t(N) + int64_t(s) * T + t) * D + c), v);
#pragma unroll
    for (int i = 0; i < kCols; ++i) acc[i] += v[i];
  }
  if constexpr (OUT_DT != kDtF32) {
    uint4 o;
    o.x = f32_to_half_bits<OUT_DT>(acc[0]) | (f32_to_half_bits<OUT_DT>(acc[1]) << 16);
    o.y = f32_to_half_bits<OUT_DT>(acc[2]) | (f32_to_half_bits<OUT_DT>(acc[3]) << 16);
    o.z = f32_to_half_bits<OUT_DT>(acc[4]) | (f32_to_half_bits<OUT_DT>(acc[5]) << 16);
    o.w = f32_to_half_bits<OUT_DT>(acc[6]) | (f32_to_half_bits<OUT_DT>(acc[7]) << 16);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + int64_t(t) * D + c) = o;
  } else {
    float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(y) + int64_t(t) * D + c);
    q[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    q[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

void launch_combine(const moe_layer_desc *d, int32_t T, const void *y_sorted, bool ys_bf16,
                    const int32_t *inv_order, const float *topk_w, void *y, int32_t out_dtype,
                    void *stream, StageMarker *mk) {
  const int N = T * d->top_k, D = d->d_model;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(T, (D + kThreads * kCols - 1) / (kThreads * kCols));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, y_sorted, inv_order, topk_w, T, d->top_k, d->n_shared,
                       N, D, y);
  };
  auto by_out = [&](auto ys_tag) {
    constexpr bool YS = decltype(ys_tag)::value;
    if (out_dtype == MOE_DT_BF16) go(combine_kernel<YS, kDtBF16>);
    else if (out_dtype == MOE_DT_F16) go(combine_kernel<YS, kDtF16>);
    else go(combine_kernel<YS, kDtF32>);
  };
  if (ys_bf16) by_out(std::true_type{});
  else by_out(std::false_type{});
  if (mk) mk->mark("combine");
}

}  // namespace moe
