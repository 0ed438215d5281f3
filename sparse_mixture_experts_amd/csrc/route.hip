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
// +0, and the bias is added last.
//
// The chunk partials are independent, so they are computed in parallel:
// kernel 1 gives each thread one chunk of 8 experts for TT tokens (8*TT
// independent fma chains; one 16-byte router load per column feeds 8*TT fmas;
// the token columns come from LDS as fp32).  When one workgroup holds every
// chunk of its (token, expert) block (large T), it adds the partials in chunk
// order from LDS and writes logits; for small T the chunks are spread over
// more workgroups to spread the router-weight reads over many CUs, and the
// raw partials go to a small global buffer.  Kernel 2 takes one wave per
// token: it adds any remaining partials in chunk order, then selects the top-k
// with a butterfly argmax per slot and computes the fp32 softmax weights.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "dispatch_tiny.h"
#include "f16_stage.h"
#include "launch.h"
#include "moe_internal.h"
#include "select_token.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

constexpr int kXsPad = 8;
// Up to this many tokens the logits run as chunk partials (one wave per (64
// experts, chunk, 8 tokens)), summed in chunk order by the selection kernel.
constexpr int kChunkRouterMaxT = 512;

// LDS index of staged column k (relative to the block's first column), token t.
template <int TT>
__device__ __forceinline__ int xs_at(int k, int t) {
  return (k / kChunk) * (kChunk * TT + kXsPad) + (k % kChunk) * TT + t;
}


// Eight consecutive router weights as fp32.
template <int DT>
__device__ __forceinline__ void load_w8(const void *w, int64_t i, float o[8]) {
  if constexpr (DT != kDtF32) {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(w) + i);
    o[0] = half_lo<DT>(u.x); o[1] = half_hi<DT>(u.x); o[2] = half_lo<DT>(u.y); o[3] = half_hi<DT>(u.y);
    o[4] = half_lo<DT>(u.z); o[5] = half_hi<DT>(u.z); o[6] = half_lo<DT>(u.w); o[7] = half_hi<DT>(u.w);
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(w) + i);
    const float4 a = p[0], b = p[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
}

// Chunk partials.  Block (tb, eb, cb): tokens tb*TT.., experts eb*EPB.., chunks
// cb*CPB..; thread = (chunk lane tid / EO, expert octet tid % EO).
// FULL: the block holds all chunks -> logits[T][E]; else partials[C][T][E].
template <int DT, int TT, int CPB>
__global__ __launch_bounds__(kThreads) void route_partials_kernel(
    const void *__restrict__ x, const void *__restrict__ wr, const float *__restrict__ bias, int T, int D,
    int E, int full, float *__restrict__ out) {
  constexpr int EO = kThreads / CPB;  // expert octets per block
  constexpr int EPB = EO * 8;         // experts per block
  extern __shared__ float lds[];
  // xs: token columns, [CPB][64 + pad][TT]: each chunk's block is padded by 8
  // floats so that the chunk lanes of a wave, which read 64 columns apart,
  // hit different LDS banks.
  float *xs = lds;
  float *part = lds;  // [CPB][TT][EPB] chunk partials, overlaying xs once it is consumed

  const int tid = threadIdx.x, cl = tid / EO, eo = tid % EO;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * EPB, c0 = blockIdx.z * CPB;
  const int C = (D + kChunk - 1) / kChunk;
  const int nt = min(TT, T - t0);
  const int kbeg = c0 * kChunk, kend = min(D, (c0 + CPB) * kChunk);

  for (int q = tid; q < (kend - kbeg) * TT; q += kThreads) {
    const int k = q / TT, t = q % TT;
    xs[xs_at<TT>(k, t)] = t < nt ? load_act<DT>(x, int64_t(t0 + t) * D + kbeg + k) : 0.0f;
  }
  __syncthreads();

  const int c = c0 + cl;
  const int e = e0 + eo * 8;
  const bool active = c < C && e < E;
  float p[TT][8];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) p[t][j] = 0.0f;
  if (active) {
    const int kc = c * kChunk, n = min(D, kc + kChunk) - kc;
    // 8 router columns of 8 experts are loaded before they are used, so the
    // loads of a step overlap each other; experts past E read as 0.
    const bool vec = (E % 8) == 0;
    for (int k8 = 0; k8 < n; k8 += 8) {
      float w[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t base = int64_t(kc + k8 + u) * E + e;
        if (k8 + u < n && vec) {
          load_w8<DT>(wr, base, w[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[u][j] = (k8 + u < n && e + j < E) ? load_act<DT>(wr, base + j) : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k8 + u < n) {
          const float *xk = xs + xs_at<TT>(kc + k8 + u - kbeg, 0);
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            const float xv = xk[t];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[t][j] = __builtin_fmaf(xv, w[u][j], p[t][j]);
          }
        }
      }
    }
  }
  __syncthreads();  // everyone is done with xs, which part overlays
  if (active) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) part[(cl * TT + t) * EPB + eo * 8 + j] = p[t][j];
  }
  __syncthreads();

  if (full) {
    // All chunks are here: chunk-ordered sum, then the bias.
    for (int q = tid; q < TT * EPB; q += kThreads) {
      const int t = q / EPB, el = q % EPB;
      if (t >= nt || e0 + el >= E) continue;
      float acc = 0.0f;
      for (int cc = 0; cc < C; ++cc) acc = acc + part[(cc * TT + t) * EPB + el];
      if (bias) acc = acc + bias[e0 + el];
      out[int64_t(t0 + t) * E + e0 + el] = acc;
    }
  } else {
    for (int q = tid; q < CPB * TT * EPB; q += kThreads) {
      const int cc = q / (TT * EPB), t = (q / EPB) % TT, el = q % EPB;
      if (c0 + cc >= C || t >= nt || e0 + el >= E) continue;
      out[(int64_t(c0 + cc) * T + t0 + t) * E + e0 + el] = part[q];
    }
  }
}

// Chunk partials for small T: one wave per (64 experts, one chunk, TT
// tokens), lane = expert.  Each lane runs the chunk's fma chain for its
// expert and TT tokens; a wave's router loads are coalesced (64 consecutive
// experts of one column) and the token values, staged in LDS, are the same
// for every lane.  Output partials[C][T][E] (no bias).
template <int DT, int TT>
__global__ __launch_bounds__(kWave) void route_chunk_kernel(const void *__restrict__ x, const void *__restrict__ wr,
                                                            int T, int D, int E, float *__restrict__ out) {
  __shared__ float xs[kChunk][TT];
  const int lane = threadIdx.x, e = blockIdx.x * kWave + lane, c = blockIdx.y, t0 = blockIdx.z * TT;
  const int kc = c * kChunk, n = min(kChunk, D - kc), nt = min(TT, T - t0);
  const int ec = min(e, E - 1);
  // the whole chunk's router column is loaded at once, in flight together
  // with the token values (one memory round trip)
  float w[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u) w[u] = load_act<DT>(wr, int64_t(kc + min(u, n - 1)) * E + ec);
#pragma unroll
  for (int t = 0; t < TT; ++t)
    xs[lane][t] = (lane < n && t < nt) ? load_act<DT>(x, int64_t(t0 + t) * D + kc + lane) : 0.0f;
  __syncthreads();
  float p[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) p[t] = 0.0f;
#pragma unroll
  for (int u = 0; u < kChunk; ++u) {
    if (u < n) {
#pragma unroll
      for (int t = 0; t < TT; ++t) p[t] = __builtin_fmaf(xs[u][t], w[u], p[t]);
    }
  }
  if (e < E) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t < nt) out[(int64_t(c) * T + t0 + t) * E + e] = p[t];
  }
}

// With x16 set (affine layers, d <= 4096), the wave also writes the token's
// fp16 staging row for the expert GEMMs; its loads go out with the others.
// With dsp.order set (all tokens in this one workgroup, T*k <= 128), the
// selected ids also go to LDS and wave 0 then performs the dispatch.
template <int MPL>
__global__ __launch_bounds__(kThreads) void route_select_kernel(const float *__restrict__ in, int n_chunks,
                                                                const float *__restrict__ bias, int T, int E,
                                                                int K, int renorm, int32_t *__restrict__ idx_out,
                                                                float *__restrict__ w_out, const uint16_t *x, int D,
                                                                uint16_t *x16, int8_t *xsh, int x_f16, XgOut xo,
                                                                FusedDispatch dsp) {
  __shared__ int32_t s_f[kTinyFusedMaxN];
  __shared__ int32_t s_cnt[kMaxExperts];
  const int t = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t < T) select_token<MPL>(t, in, n_chunks, bias, T, E, K, renorm, idx_out, w_out, x, D, x16, xsh, x_f16,
                               xo, dsp.order ? s_f : nullptr);
  if (dsp.order) {
    __syncthreads();
    if (threadIdx.x < kWave)
      tiny_dispatch<kTinyFusedMaxN / kWave>(s_f, T * K, K, E, dsp.S, T, dsp.tile_rows, dsp.tr, dsp.order, dsp.inv_order, dsp.row_map,
                    dsp.expert_off, dsp.tile_off, dsp.counters, dsp.act_items, dsp.tiles, s_cnt);
  }
}

void launch_select(const float *in, int n_chunks, const float *bias, int T, int E, int K, int renorm,
                   int32_t *idx, float *w, const void *x, int D, void *x16, int8_t *xsh, bool x_f16, XgOut xo,
                   const FusedDispatch &dsp, hipStream_t s) {
  const dim3 grid((T + kThreads / kWave - 1) / (kThreads / kWave)), block(kThreads);
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  uint16_t *x16o = static_cast<uint16_t *>(x16);
  auto go = [&](auto kern) {
    launch(kern, grid, block, 0, s, in, n_chunks, bias, T, E, K, renorm, idx, w, xb, D, x16o, xsh,
                       int(x_f16), xo, dsp);
  };
  if (E <= 64) go(route_select_kernel<1>);
  else if (E <= 128) go(route_select_kernel<2>);
  else if (E <= 256) go(route_select_kernel<4>);
  else if (E <= 512) go(route_select_kernel<8>);
  else go(route_select_kernel<16>);
}

// Returns true when one block held every chunk (the output is logits).
template <int DT, int TT, int CPB>
bool launch_partials(const void *x, const void *wr, const float *bias, int T, int D, int E, float *out,
                     hipStream_t s) {
  constexpr int EPB = (kThreads / CPB) * 8;
  const int C = (D + kChunk - 1) / kChunk;
  const dim3 grid((T + TT - 1) / TT, (E + EPB - 1) / EPB, (C + CPB - 1) / CPB);
  const int full = grid.z == 1;
  const size_t lds = std::max(size_t(CPB) * (kChunk * TT + kXsPad), size_t(CPB) * TT * EPB) * sizeof(float);
  if (lds > 64 * 1024) {
    // Above the default dynamic-LDS limit (gfx950 has 160 KB per CU): raise it
    // once per process for this kernel.
    static const bool raised = [&] {
      return hipFuncSetAttribute(reinterpret_cast<const void *>(&route_partials_kernel<DT, TT, CPB>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) == hipSuccess;
    }();
    (void)raised;
  }
  launch((route_partials_kernel<DT, TT, CPB>), grid, dim3(kThreads), lds, s, x, wr, bias, T, D,
                     E, full, out);
  return full;
}

}  // namespace

int64_t route_scratch_floats(const moe_layer_desc *d, int32_t T) {
  // Covers every T' <= T: below 64 tokens (and at any T when C > 32) the
  // chunk partials, C per (token, expert), go through the workspace.
  const int64_t C = (d->d_model + kChunk - 1) / kChunk;
  const int64_t t_split = C <= 32 ? std::min<int64_t>(T, kChunkRouterMaxT) : int64_t(T);
  int64_t n = std::max<int64_t>(int64_t(T) * d->n_experts, C * t_split * d->n_experts);
  if (route_mfma_applies(d, T)) n = std::max(n, route_mfma_scratch_floats(d, T));
  return n;
}

bool route_writes_x16(const moe_layer_desc *d) {
  return affine(d) && d->d_model <= kRowF16MaxD;
}

bool route_fuses_dispatch(const moe_layer_desc *d, int32_t T) {
  return T <= kThreads / kWave && int64_t(T) * d->top_k <= kTinyFusedMaxN && !route_mfma_applies(d, T);
}

int launch_route_chunks_t1(const moe_layer_desc *d, const void *x, const void *w_router, float *partials,
                           void *stream, StageMarker *mk) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_model, E = d->n_experts, C = (D + kChunk - 1) / kChunk;
  const dim3 grid((E + kWave - 1) / kWave, C, 1);
  if (d->act_dtype == MOE_DT_BF16)
    launch((route_chunk_kernel<kDtBF16, 1>), grid, dim3(kWave), 0, s, x, w_router, 1, D, E, partials);
  else if (d->act_dtype == MOE_DT_F16)
    launch((route_chunk_kernel<kDtF16, 1>), grid, dim3(kWave), 0, s, x, w_router, 1, D, E, partials);
  else
    launch((route_chunk_kernel<kDtF32, 1>), grid, dim3(kWave), 0, s, x, w_router, 1, D, E, partials);
  if (mk) mk->mark("route_logits");
  return C;
}

void launch_route(const moe_layer_desc *d, int32_t T, const void *x, const void *w_router,
                  const float *bias, int32_t *idx, float *w, float *scratch, void *x16, int8_t *xsh,
                  uint16_t *xg, const FusedDispatch &dsp_in, void *stream, StageMarker *mk,
                  const void *router_packed) {
  if (!route_writes_x16(d)) x16 = nullptr, xsh = nullptr;
  const XgOut xo = xg_out(d, x16 ? xg : nullptr);
  FusedDispatch dsp = dsp_in;
  if (!route_fuses_dispatch(d, T)) dsp.order = nullptr;
  if (route_mfma_applies(d, T)) {
    const bool counts = dsp.counts && route_counts_dispatch(d, T);
    launch_route_mfma(d, T, x, w_router, bias, idx, w, scratch, x16, xsh, xo, stream, mk, counts ? dsp.counts : nullptr,
                      counts ? int(dispatch_segment_slots(d, T)) : 0, router_packed);
    return;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_model, E = d->n_experts;
  const int C = (D + kChunk - 1) / kChunk;
  // Up to 512 tokens: one wave per (64 experts, chunk, 2 or 4 tokens) for
  // many parallel fma chains, the partials summed by the selection kernel.  Beyond
  // (when the matrix-core router does not apply): 8 tokens per block with
  // every chunk of the block on chip; with d_model > 2048 one token per
  // block, 2 chunks per block.
  int n_chunks = C;
  auto logits = [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (T == 1) {
      // one token: one chain per lane (no idle token slots)
      const dim3 grid((E + kWave - 1) / kWave, C, 1);
      launch((route_chunk_kernel<DT, 1>), grid, dim3(kWave), 0, s, x, w_router, T, D, E, scratch);
    } else if (T <= kChunkRouterMaxT) {
      // tokens per wave: 2 when every lane has an expert, else 4 (more
      // chains per loaded router column); measured against 8: 32-token
      // decode 8.6 -> 5.0 us, the skewed 256-token layer 9.9 -> 7.6 us, the
      // dense 8-expert layer 10.8 -> 9.6 us with 4
      if (E >= kWave) {
        const dim3 grid((E + kWave - 1) / kWave, C, (T + 1) / 2);
        launch((route_chunk_kernel<DT, 2>), grid, dim3(kWave), 0, s, x, w_router, T, D, E, scratch);
      } else {
        const dim3 grid((E + kWave - 1) / kWave, C, (T + 3) / 4);
        launch((route_chunk_kernel<DT, 4>), grid, dim3(kWave), 0, s, x, w_router, T, D, E, scratch);
      }
    } else if (C <= 32) {
      launch_partials<DT, 8, 32>(x, w_router, bias, T, D, E, scratch, s);
      n_chunks = 0;
    } else {
      n_chunks = launch_partials<DT, 1, 2>(x, w_router, bias, T, D, E, scratch, s) ? 0 : C;
    }
  };
  if (d->act_dtype == MOE_DT_BF16) logits(std::integral_constant<int, kDtBF16>{});
  else if (d->act_dtype == MOE_DT_F16) logits(std::integral_constant<int, kDtF16>{});
  else logits(std::integral_constant<int, kDtF32>{});
  if (mk) mk->mark("route_logits");
  launch_select(scratch, n_chunks, bias, T, E, d->top_k, d->renormalize, idx, w, x, D, x16, xsh,
                d->act_dtype == MOE_DT_F16, xo, dsp, s);
  if (mk) mk->mark(dsp.order ? "route_select_dispatch" : "route_select");
}

}  // namespace moe
