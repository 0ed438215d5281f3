// select_token.h -- one wave selects one token's experts from its router
// logits (or the chunk partials of the canonical order): top-k by logit with
// the lower expert index first on ties, then the fp32 softmax weights,
// renormalised over the k winners when asked.
#pragma once

#include "device_common.h"
#include "f16_stage.h"

namespace moe {
namespace {

// One wave per token: logits (summing chunk partials when n_chunks > 0),
// top-k, softmax.  Each lane keeps the logits of experts lane + 64*m, m < MPL.
// The per-token part of the selection kernel (one wave).
template <int MPL>
__device__ __forceinline__ void select_token(int t, const float *__restrict__ in, int n_chunks,
                                             const float *__restrict__ bias, int T, int E, int K, int renorm,
                                             int32_t *__restrict__ idx_out, float *__restrict__ w_out,
                                             const uint16_t *x, int D, uint16_t *x16, int8_t *xsh, bool x_f16,
                                             XgOut xo, int32_t *s_f) {
  // chunk partials per load batch: about 64 loads in flight per lane
  constexpr int CB = MPL >= 64 ? 1 : 64 / MPL;
  const int lane = lane_id();
  RowF16 xr;
  if (x16) row_f16_load(x + int64_t(t) * D, D, xr);
  float l[MPL];
  if (n_chunks == 0) {
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
      const int e = lane + kWave * m;
      l[m] = e < E ? in[int64_t(t) * E + e] : -INFINITY;
    }
  } else {
    float acc[MPL];
#pragma unroll
    for (int m = 0; m < MPL; ++m) acc[m] = 0.0f;
    for (int c0 = 0; c0 < n_chunks; c0 += CB) {
      float pv[CB][MPL];
#pragma unroll
      for (int u = 0; u < CB; ++u)
#pragma unroll
        for (int m = 0; m < MPL; ++m) {
          const int e = min(lane + kWave * m, E - 1), c = min(c0 + u, n_chunks - 1);
          pv[u][m] = in[(int64_t(c) * T + t) * E + e];
        }
      // chunk order
#pragma unroll
      for (int u = 0; u < CB; ++u)
        if (c0 + u < n_chunks) {
#pragma unroll
          for (int m = 0; m < MPL; ++m) acc[m] = acc[m] + pv[u][m];
        }
    }
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
      const int e = lane + kWave * m;
      l[m] = e < E ? (bias ? acc[m] + bias[e] : acc[m]) : -INFINITY;
    }
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_l = 0.0f, top = 0.0f;
  for (int j = 0; j < K; ++j) {
    float bv;
    const int be = wave_argmax<MPL>(l, E, taken, bv);
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    if (j == 0) top = bv;
    if (lane == j) { my_e = be; my_l = bv; }
  }
  // fp32 softmax over all E logits (the top-1 logit is the maximum).
  float z = 0.0f;
#pragma unroll
  for (int m = 0; m < MPL; ++m)
    if (lane + kWave * m < E) z += expf(l[m] - top);
  z = wave_sum(z);
  const float p = expf(my_l - top) / z;
  float w = p;
  if (renorm) {
    float psum = 0.0f;
    for (int j = 0; j < K; ++j) psum = psum + read_lane(p, j);
    w = p / psum;
  }
  if (lane < K) {
    idx_out[int64_t(t) * K + lane] = my_e;
    w_out[int64_t(t) * K + lane] = w;
    if (s_f) s_f[t * K + lane] = my_e;
  }
  if (x16) row_f16_store(xr, D, x16 + int64_t(t) * D, xsh + t, x_f16, xo, t);
}

}  // namespace
}  // namespace moe
