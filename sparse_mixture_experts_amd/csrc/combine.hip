// combine.hip -- score-weighted unsort of the expert outputs.
//
// y[t] = sum_j w[t][j] * y_sorted[inv_order[t*k + j]] + sum_s y_shared_s[t]:
// the weighted sum of "perf(moe): fused MoE expert decode kernel" ("What it
// does") gathered through inv_order as in DS4Server #112's _scatter_unsort.
// A gather per token instead of the PRD's atomic scatter-add keeps the fp32
// summation order fixed (slot order), so results are deterministic.  Expert
// outputs arrive as fp32 rows, as fp16 rows with one power-of-two exponent
// per 64 columns, or (down reduction split) as fp32 partial rows that are
// first summed in part order.
#include <stdexcept>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 8;  // columns per thread (one 16-byte fp16 load, two fp32 ones)

// Eight consecutive expert-output values, as loaded (fp16: one 16-byte load
// and the row's exponent for these columns; fp32: two 16-byte loads) and as
// fp32.
template <bool F16E>
struct Row8 {
  uint4 u[F16E ? 1 : 2];
  int sh;
};
template <bool F16E>
__device__ __forceinline__ Row8<F16E> load8(const void *ys, const int8_t *ys_sh, int64_t row, int D, int c) {
  Row8<F16E> r;
  const int64_t i = row * D + c;
  if constexpr (F16E) {
    r.u[0] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(ys) + i);
    r.sh = ys_sh[row * (D / kYsBlock) + c / kYsBlock];
  } else {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const float *>(ys) + i);
    r.u[0] = q[0];
    r.u[1] = q[1];
    r.sh = 0;
  }
  return r;
}
__device__ __forceinline__ float f16_lo(uint32_t u) { return float(__builtin_bit_cast(_Float16, uint16_t(u))); }
__device__ __forceinline__ float f16_hi(uint32_t u) { return float(__builtin_bit_cast(_Float16, uint16_t(u >> 16))); }
template <bool F16E>
__device__ __forceinline__ void widen8(const Row8<F16E> &r, float v[8]) {
  if constexpr (F16E) {
    const uint4 u = r.u[0];
    const float m = __uint_as_float(uint32_t(127 + r.sh) << 23);  // 2^sh
    v[0] = f16_lo(u.x) * m; v[1] = f16_hi(u.x) * m; v[2] = f16_lo(u.y) * m; v[3] = f16_hi(u.y) * m;
    v[4] = f16_lo(u.z) * m; v[5] = f16_hi(u.z) * m; v[6] = f16_lo(u.w) * m; v[7] = f16_hi(u.w) * m;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v[4 * h] = __uint_as_float(r.u[h].x); v[4 * h + 1] = __uint_as_float(r.u[h].y);
      v[4 * h + 2] = __uint_as_float(r.u[h].z); v[4 * h + 3] = __uint_as_float(r.u[h].w);
    }
  }
}

// Adds the partial rows 1 .. parts-1 of the fp32 row `row`, columns c .. c+7.
__device__ __forceinline__ void add_parts(const void *ys, int64_t row, int D, int c, int parts,
                                          int64_t part_rows, float v[8]) {
  for (int z = 1; z < parts; ++z) {
    float q[kCols];
    widen8<false>(load8<false>(ys, nullptr, z * part_rows + row, D, c), q);
#pragma unroll
    for (int i = 0; i < kCols; ++i) v[i] += q[i];
  }
}

// Block (t, cb): token t, columns cb*256*8 ..; each thread 8 columns.  The
// token's slot positions and weights are uniform (scalar loads); then all
// slot rows of a thread (up to 16 fp16 or 8 fp32 rows per round) are in
// flight together before they are summed in slot order; SL slots per round
// (the launch picks the smallest that covers k, up to 16 fp16 or 8 fp32
// rows).  parts > 1 (fp32 rows only): partial rows part_rows rows apart.
template <bool F16E, int OUT_DT, int SL>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void *__restrict__ ys,
                                                           const int8_t *__restrict__ ys_sh,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ w, int T, int K, int S,
                                                           int N, int D, int parts, int64_t part_rows,
                                                           void *__restrict__ y) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * kCols;
  if (c >= D) return;
  float acc[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
  constexpr int kSlots = SL;
  for (int j0 = 0; j0 < K; j0 += kSlots) {
    Row8<F16E> r[kSlots];
    float wj[kSlots];
    int rowj[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int j = min(j0 + u, K - 1);
      const int p = inv[int64_t(t) * K + j];
      const bool ok = j0 + u < K && unsigned(p) < unsigned(N);
      wj[u] = ok ? w[int64_t(t) * K + j] : 0.f;
      rowj[u] = ok ? p : 0;
      r[u] = load8<F16E>(ys, ys_sh, rowj[u], D, c);
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
      if (j0 + u < K) {
        float v[kCols];
        widen8<F16E>(r[u], v);
        if constexpr (!F16E) add_parts(ys, rowj[u], D, c, parts, part_rows, v);
#pragma unroll
        for (int i = 0; i < kCols; ++i) acc[i] += wj[u] * v[i];
      }
  }
  for (int s = 0; s < S; ++s) {
    float v[kCols];
    const int64_t row = int64_t(N) + int64_t(s) * T + t;
    widen8<F16E>(load8<F16E>(ys, ys_sh, row, D, c), v);
    if constexpr (!F16E) add_parts(ys, row, D, c, parts, part_rows, v);
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

void launch_combine(const moe_layer_desc *d, int32_t T, const void *y_sorted, const int8_t *ys_sh,
                    const int32_t *inv_order, const float *topk_w, void *y, int32_t out_dtype,
                    void *stream, StageMarker *mk, int parts) {
  const int N = T * d->top_k, D = d->d_model;
  if (parts > 1 && ys_sh) throw std::invalid_argument("combine: partial rows are fp32");
  if (ys_sh && D % kYsBlock) throw std::invalid_argument("combine: fp16 rows need d_model % 64 == 0");
  const int64_t part_rows = int64_t(N) + int64_t(d->n_shared) * T;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(T, (D + kThreads * kCols - 1) / (kThreads * kCols));
  auto go = [&](auto kern) {
    launch(kern, grid, dim3(kThreads), 0, s, y_sorted, ys_sh, inv_order, topk_w, T, d->top_k,
                       d->n_shared, N, D, parts, part_rows, y);
  };
  const int K = d->top_k;
  auto by_out = [&](auto ys_tag, auto sl_tag) {
    constexpr bool F16E = decltype(ys_tag)::value;
    constexpr int SL = decltype(sl_tag)::value;
    if (out_dtype == MOE_DT_BF16) go(combine_kernel<F16E, kDtBF16, SL>);
    else if (out_dtype == MOE_DT_F16) go(combine_kernel<F16E, kDtF16, SL>);
    else go(combine_kernel<F16E, kDtF32, SL>);
  };
  using S4 = std::integral_constant<int, 4>;
  using S8 = std::integral_constant<int, 8>;
  using S12 = std::integral_constant<int, 12>;
  using S16 = std::integral_constant<int, 16>;
  if (ys_sh) {
    if (K <= 4) by_out(std::true_type{}, S4{});
    else if (K <= 8) by_out(std::true_type{}, S8{});
    else if (K <= 12) by_out(std::true_type{}, S12{});
    else by_out(std::true_type{}, S16{});
  } else {
    if (K <= 4) by_out(std::false_type{}, S4{});
    else by_out(std::false_type{}, S8{});
  }
  if (mk) mk->mark("combine");
}

}  // namespace moe
