// ffn_gemv.hip -- grouped expert FFN on the vector units, for the layers the
// matrix-core kernels do not take: fp32 activations, or dense bf16/fp16
// layers whose d_model or d_ff is not a multiple of 64.  (Affine layers
// always have 16-bit activations and 64-multiple dims, so they always run on
// the matrix cores.)
//
// "SwitchGLU: grouped-expert Metal kernels" (ml-explore/mlx-lm #2044),
// section "What": slots are grouped by expert across tokens so each expert's
// weights are read once per group of rows instead of once per (token, slot);
// gate and up are computed in one pass.  "perf(moe): fused MoE expert decode
// kernel" (lablup/mlxcel #275), "What it does": SwiGLU, down projection.
//
// One workgroup takes one plan item (an expert and its sorted rows) and a
// block of output columns.  Up to MR of the item's rows are staged in LDS;
// each wave computes whole output columns: its 64 lanes split the reduction
// dim into 8-element pieces (one 32-bit word of 4-bit codes, or 16/32 bytes
// of dense weights, per lane and step, so a wave reads 256..2048 contiguous
// bytes of a weight row per step), dequantises once, and applies the piece to
// all staged rows; a butterfly sum finishes each dot product.
#include "device_common.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMR = 8;        // rows per pass (register accumulators)
constexpr int kNB = 16;       // output columns per workgroup (4 per wave)
constexpr int kThreads = 256;

// Weights k..k+7 of global row `row` (expert-major row index) of a [.][K] matrix.
template <int DT>
__device__ __forceinline__ void load_w8(const void *__restrict__ w, const uint16_t *__restrict__ sc,
                                        const uint16_t *__restrict__ bi, int64_t row, int K, int k,
                                        float out[8]) {
  if constexpr (DT == kDtF32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(w) + row * K + k);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(w) + row * K + k);
    out[0] = half_lo<DT>(u.x); out[1] = half_hi<DT>(u.x); out[2] = half_lo<DT>(u.y); out[3] = half_hi<DT>(u.y);
    out[4] = half_lo<DT>(u.z); out[5] = half_hi<DT>(u.z); out[6] = half_lo<DT>(u.w); out[7] = half_hi<DT>(u.w);
  }
}

// Eight staged activations (fp32, or 16-bit bits in LDS) as fp32.
template <int DT>
__device__ __forceinline__ void lds_x8(const void *xs, int idx, float out[8]) {
  if constexpr (DT != kDtF32) {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xs) + idx);
    out[0] = half_lo<DT>(u.x); out[1] = half_hi<DT>(u.x); out[2] = half_lo<DT>(u.y); out[3] = half_hi<DT>(u.y);
    out[4] = half_lo<DT>(u.z); out[5] = half_hi<DT>(u.z); out[6] = half_lo<DT>(u.w); out[7] = half_hi<DT>(u.w);
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(xs) + idx);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// Stage `mr` rows of length K into LDS; row m comes from src row src_row(m).
template <int DT, class RowOf>
__device__ __forceinline__ void stage_rows(void *xs, const void *__restrict__ src, int mr, int K,
                                           RowOf src_row) {
  // 16-byte pieces: 8 16-bit or 4 fp32 elements.
  constexpr int ESZ = DT == kDtF32 ? 4 : 2;  // element bytes
  constexpr int EPP = 16 / ESZ;
  const int ppr = K / EPP;
  for (int q = threadIdx.x; q < mr * ppr; q += blockDim.x) {
    const int m = q / ppr, c = (q % ppr) * EPP;
    const int64_t r = src_row(m);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r >= 0) v = *reinterpret_cast<const uint4 *>(static_cast<const char *>(src) + (r * K + c) * ESZ);
    *reinterpret_cast<uint4 *>(static_cast<char *>(xs) + (int64_t(m) * K + c) * ESZ) = v;
  }
}

struct GateUpArgs {
  const void *x;
  const int32_t *row_map;
  int T, N, D, F, E, fused, round_ops, geglu, MR;
  const void *wg;
  const uint16_t *sg, *bg;
  const void *wu;
  const uint16_t *su, *bu;
  const int32_t *counters;
  const PlanItem *items;
  void *h;
};

template <int DT>
__global__ __launch_bounds__(kThreads) void gateup_gemv_kernel(GateUpArgs a) {
  extern __shared__ uint4 smem_v[];
  void *xs = smem_v;
  if (int(blockIdx.y) >= a.counters[0]) return;
  const PlanItem it = a.items[blockIdx.y];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int D = a.D, F = a.F;
  for (int r0 = 0; r0 < it.rows; r0 += a.MR) {
    const int mr = min(a.MR, it.rows - r0);
    __syncthreads();
    stage_rows<DT>(xs, a.x, mr, D, [&](int m) -> int64_t {
      const int p = it.row0 + r0 + m;
      const int t = p < a.N ? a.row_map[p] : (p - a.N) % a.T;
      return unsigned(t) < unsigned(a.T) ? int64_t(t) : int64_t(-1);
    });
    __syncthreads();
    for (int nq = 0; nq < kNB / 4; ++nq) {
      const int n = blockIdx.x * kNB + wave * (kNB / 4) + nq;
      if (n >= F) break;
      const int64_t rg = a.fused ? int64_t(it.expert) * 2 * F + n : int64_t(it.expert) * F + n;
      const int64_t ru = a.fused ? rg + F : rg;
      const void *wu = a.fused ? a.wg : a.wu;
      const uint16_t *su = a.fused ? a.sg : a.su, *bu = a.fused ? a.bg : a.bu;
      float ag[kMR], au[kMR];
#pragma unroll
      for (int m = 0; m < kMR; ++m) ag[m] = au[m] = 0.0f;
      for (int k = lane * 8; k < D; k += 8 * kWave) {
        float wg8[8], wu8[8];
        load_w8<DT>(a.wg, a.sg, a.bg, rg, D, k, wg8);
        load_w8<DT>(wu, su, bu, ru, D, k, wu8);
#pragma unroll
        for (int m = 0; m < kMR; ++m) {
          if (m < mr) {
            float xv[8];
            lds_x8<DT>(xs, m * D + k, xv);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              ag[m] += xv[u] * wg8[u];
              au[m] += xv[u] * wu8[u];
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kMR; ++m) {
        if (m < mr) {
          const float g = wave_sum(ag[m]), u = wave_sum(au[m]);
          if (lane == 0) {
            const float hv = glu(g, u, a.round_ops, a.geglu);
            const int64_t o = int64_t(it.row0 + r0 + m) * F + n;
            if constexpr (DT != kDtF32) static_cast<uint16_t *>(a.h)[o] = uint16_t(f32_to_half_bits<DT>(hv));
            else static_cast<float *>(a.h)[o] = hv;
          }
        }
      }
    }
  }
}

struct DownArgs {
  const void *h;
  int D, F, MR;
  const void *wd;
  const uint16_t *sd, *bd;
  const int32_t *counters;
  const PlanItem *items;
  float *y;
};

template <int DT>
__global__ __launch_bounds__(kThreads) void down_gemv_kernel(DownArgs a) {
  extern __shared__ uint4 smem_v[];
  void *hs = smem_v;
  if (int(blockIdx.y) >= a.counters[0]) return;
  const PlanItem it = a.items[blockIdx.y];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int D = a.D, F = a.F;
  for (int r0 = 0; r0 < it.rows; r0 += a.MR) {
    const int mr = min(a.MR, it.rows - r0);
    __syncthreads();
    stage_rows<DT>(hs, a.h, mr, F, [&](int m) -> int64_t { return it.row0 + r0 + m; });
    __syncthreads();
    for (int nq = 0; nq < kNB / 4; ++nq) {
      const int n = blockIdx.x * kNB + wave * (kNB / 4) + nq;
      if (n >= D) break;
      const int64_t rd = int64_t(it.expert) * D + n;
      float acc[kMR];
#pragma unroll
      for (int m = 0; m < kMR; ++m) acc[m] = 0.0f;
      for (int k = lane * 8; k < F; k += 8 * kWave) {
        float w8[8];
        load_w8<DT>(a.wd, a.sd, a.bd, rd, F, k, w8);
#pragma unroll
        for (int m = 0; m < kMR; ++m) {
          if (m < mr) {
            float hv[8];
            lds_x8<DT>(hs, m * F + k, hv);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[m] += hv[u] * w8[u];
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kMR; ++m) {
        if (m < mr) {
          const float v = wave_sum(acc[m]);
          if (lane == 0) a.y[int64_t(it.row0 + r0 + m) * D + n] = v;
        }
      }
    }
  }
}

int rows_per_pass(int K, int esz) { return max(1, min(kMR, 65536 / (K * esz))); }

template <int DT>
void launch_gemv(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                 const moe_weights *w, const int32_t *counters, const PlanItem *items, void *h,
                 float *y, hipStream_t s, StageMarker *mk) {
  const int D = d->d_model, F = d->d_ff, E = d->n_experts, S = d->n_shared;
  const int N = T * d->top_k;
  const int esz = DT == kDtF32 ? 4 : 2;
  const int max_items = min(E, N) + S;
  const moe_proj &pg = d->gate_up_fused ? w->gate_up : w->gate;
  GateUpArgs ga{x, row_map, T, N, D, F, E, d->gate_up_fused, glu_round_mode(d),
                d->activation == MOE_ACT_GEGLU, rows_per_pass(D, esz), pg.w, static_cast<const uint16_t *>(pg.scales),
                static_cast<const uint16_t *>(pg.biases), w->up.w,
                static_cast<const uint16_t *>(w->up.scales), static_cast<const uint16_t *>(w->up.biases),
                counters, items, h};
  launch((gateup_gemv_kernel<DT>), dim3((F + kNB - 1) / kNB, max_items),
                     dim3(kThreads), size_t(ga.MR) * D * esz, s, ga);
  if (mk) mk->mark("gateup_gemv");
  DownArgs da{h, D, F, rows_per_pass(F, esz), w->down.w, static_cast<const uint16_t *>(w->down.scales),
              static_cast<const uint16_t *>(w->down.biases), counters, items, y};
  launch((down_gemv_kernel<DT>), dim3((D + kNB - 1) / kNB, max_items),
                     dim3(kThreads), size_t(da.MR) * F * esz, s, da);
  if (mk) mk->mark("down_gemv");
}

}  // namespace

void launch_expert_ffn(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                       const moe_weights *w, const int32_t *counters, const PlanItem *act_items,
                       const PlanItem *tiles, int64_t max_tiles, const FfnScratch &sc, void *ys,
                       int8_t *ys_sh, void *stream, StageMarker *mk, int down_parts) {
  if (use_mfma(d)) {
    launch_expert_ffn_mfma(d, T, x, row_map, w, counters, tiles, max_tiles, sc, ys, ys_sh, stream, mk,
                           down_parts);
    return;
  }
  // The vector-unit kernels write fp32 rows (the workspace copy is fp32 for
  // the layers they serve).
  float *y_sorted = static_cast<float *>(ys);
  void *h = sc.h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->act_dtype == MOE_DT_BF16)
    launch_gemv<kDtBF16>(d, T, x, row_map, w, counters, act_items, h, y_sorted, s, mk);
  else if (d->act_dtype == MOE_DT_F16)
    launch_gemv<kDtF16>(d, T, x, row_map, w, counters, act_items, h, y_sorted, s, mk);
  else
    launch_gemv<kDtF32>(d, T, x, row_map, w, counters, act_items, h, y_sorted, s, mk);
}

}  // namespace moe
