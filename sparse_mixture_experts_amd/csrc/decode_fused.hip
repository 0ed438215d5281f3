// decode_fused.hip -- the one-token layer in three launches.
//
// "perf(moe): fused MoE expert decode kernel" (lablup/mlxcel #275), "What it
// does" and "Summary": at one token the whole expert part of the layer --
// gate/up GEMV, SwiGLU, down GEMV and the score-weighted sum -- runs with no
// host round trip and no intermediate launches per expert, spread over many
// threadgroups with in-register reductions.  "SwitchGLU: grouped-expert
// Metal kernels", "What", one-token case: gate and up in one pass, and the
// down projection with all k experts in flight.
//
// Here, after the router's chunk partials (route.hip, one wave per (64
// experts, 64 columns)):
//   1. t1_gateup_kernel, one workgroup per (slot, 8 columns of d_ff): wave 0
//      selects the token's experts from the chunk partials (the same
//      canonical-order sums and selection as the router's own selection
//      kernel), wave 1 stages x as fp16 with one power-of-two exponent, then
//      the four waves split the reduction over d_model for the slot's 8 gate
//      and 8 up rows; partial sums are added in wave order and the GLU
//      writes h (fp32, true values).  No dispatch is needed: slot j of the
//      token is expert topk[j], rows = the token.
//   2. t1_down_combine_kernel, one workgroup per 16 output columns: the h
//      rows of all slots are staged as fp16 (one exponent per row), each wave
//      runs the down rows of its slots (all slots in flight at once) and
//      scales them by the slot weight; the waves' sums are added in wave
//      order and y is written in the output dtype.
// At one token the matrix cores would multiply 16 rows for one: both kernels
// are dequant-GEMVs instead (slab_dot): code pairs under the fp16 exponent
// of 1024 meet activation pairs in v_dot2_f32_f16, the affine scale and bias
// are applied per slab in fp32, and the row's four lanes are summed with
// cross-lane swaps.  (Measured against the same kernels on 16x16x32 MFMA
// slabs, 4-bit codes: selection + gate/up 10.4 -> 10.2 us, down + combine
// 10.6 -> 9.7 us; the one-token layer 23.7 -> 22.6 us, and 28.6 -> 26.3 us
// with 8-bit codes.)
#include <hip/hip_runtime.h>

#include "dequant_f16.h"
#include "device_common.h"
#include "f16_stage.h"
#include "launch.h"
#include "moe_internal.h"
#include "select_token.h"

namespace moe {
namespace {

constexpr int kSlab = 128;        // reduction elements per slab
constexpr int kGUWaves = 4;       // gate/up: the reduction split over the workgroup's waves
constexpr int kDNWaves = 8;       // down: slots spread over the workgroup's waves
constexpr int kT1MaxD = 4096;     // d_model of the staging row
constexpr int kT1MaxF = 2048;     // d_ff held in registers by the down waves (16 slabs)
constexpr int kT1MaxHStage = 28672;  // (k + shared) * d_ff fp16 values staged per down workgroup (56 KB)
constexpr int kT1HPieces = 7;        // 8-value h pieces per down thread: 7 * 512 * 8 >= kT1MaxHStage

struct T1Args {
  const float *partials;  // router chunk partials [C][1][E]
  int n_chunks;
  const float *bias;      // [E] or null
  int E, K, S, renorm;
  const uint16_t *x;      // [D] bf16 (fp16 when x_f16)
  int x_f16;
  int D, F, fused, round_ops, geglu, gsize, half_f16;
  const uint32_t *wg;     // gate (or gate_up) codes
  const uint16_t *sg, *bg;
  const uint32_t *wu;     // up codes (separate layout)
  const uint16_t *su, *bu;
  const uint32_t *wd;     // down codes
  const uint16_t *sd, *bd;
  int32_t *idx;           // [K] selected experts (written by workgroup (0, 0))
  float *wt;              // [K] their weights
  float *h;               // [K + S][F] fp32
  float *hmax;            // [K + S][F / 8] largest |h| of each 8-column block
  void *y;                // [D] in out_dtype
  int out_dtype;
};

// Slab s of weight row `row` (codes and the scale / bias of this lane's 32
// elements); slabs past the row's end read a clamped address and get zero
// scales, so they contribute nothing.
template <int QB>
__device__ __forceinline__ void load_row_slab(const uint32_t *wrow, const uint16_t *sp, const uint16_t *bp, int nre,
                                              int K, int gsize, int s, int lg, bool valid, uint4 (&wq)[QB / 4],
                                              uint16_t &sr, uint16_t &br) {
  const int KW = K * QB / 32, G = K / gsize;
  const int w = min(s * (kSlab * QB / 32) + lg * QB, KW - QB);
#pragma unroll
  for (int v = 0; v < QB / 4; ++v) wq[v] = *reinterpret_cast<const uint4 *>(wrow + w + 4 * v);
  const int gl = (s * kSlab + lg * 32) / gsize;
  const int g = min(gl, G - 1);
  const uint16_t sv = sp[int64_t(g) * nre], bv = bp[int64_t(g) * nre];
  const bool ok = valid && gl < G;
  sr = ok ? sv : uint16_t(0);
  br = ok ? bv : uint16_t(0);
}

// Dequant-GEMV of one slab: this lane's 32 codes of its weight row against
// the 32 staged activations (staging order e0,e4,e1,e5,e2,e6,e3,e7 in every
// block of 8).  Each code pair goes under the fp16 exponent of 1024 (1024 + q
// exact, or 1024 + 16q for the 4-bit codes in bits 4-7 of a byte) and meets
// its activation pair in v_dot2_f32_f16; returns sum q*x in `qx` and sum x in
// `sx`, so that the slab's share of the row's dot product is s*qx + b*sx
// with the group's scale and bias in fp32.
template <int QB>
__device__ __forceinline__ void slab_dot(const uint4 (&wq)[QB / 4], const uint16_t *act, uint32_t magic, float &qx,
                                         float &sx) {
  const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float a1 = 0.f, a16 = 0.f, s1 = 0.f, s16 = 0.f;  // code pairs taken as 1024 + q / 1024 + 16q, and their x sums
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 xv = *reinterpret_cast<const uint4 *>(act + j * 8);
    const h2 X0 = __builtin_bit_cast(h2, xv.x), X1 = __builtin_bit_cast(h2, xv.y);
    const h2 X2 = __builtin_bit_cast(h2, xv.z), X3 = __builtin_bit_cast(h2, xv.w);
    if constexpr (QB == 4) {
      const uint32_t w = j == 0 ? wq[0].x : j == 1 ? wq[0].y : j == 2 ? wq[0].z : wq[0].w;
      const uint32_t w8 = w >> 8;
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (w & 0x000f000fu) | magic), X0, a1, false);
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (w8 & 0x000f000fu) | magic), X2, a1, false);
      a16 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (w & 0x00f000f0u) | magic), X1, a16, false);
      a16 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (w8 & 0x00f000f0u) | magic), X3, a16, false);
      s1 = __builtin_amdgcn_fdot2(X0, one2, s1, false);
      s1 = __builtin_amdgcn_fdot2(X2, one2, s1, false);
      s16 = __builtin_amdgcn_fdot2(X1, one2, s16, false);
      s16 = __builtin_amdgcn_fdot2(X3, one2, s16, false);
    } else {
      // two words hold the block's 8 codes (see q8_words_to_f16)
      const uint4 &q = wq[j >> 1];
      const uint32_t w0 = (j & 1) ? q.z : q.x, w1 = (j & 1) ? q.w : q.y;
      const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // q0, q4, q1, q5
      const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // q2, q6, q3, q7
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, t0, 0x04010400u)), X0, a1, false);
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, t0, 0x04030402u)), X1, a1, false);
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, t1, 0x04010400u)), X2, a1, false);
      a1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, t1, 0x04030402u)), X3, a1, false);
      s1 = __builtin_amdgcn_fdot2(X0, one2, s1, false);
      s1 = __builtin_amdgcn_fdot2(X1, one2, s1, false);
      s1 = __builtin_amdgcn_fdot2(X2, one2, s1, false);
      s1 = __builtin_amdgcn_fdot2(X3, one2, s1, false);
    }
  }
  qx = (a1 - 1024.0f * s1) + (QB == 4 ? (a16 - 1024.0f * s16) * 0.0625f : 0.0f);
  sx = s1 + s16;
}

__device__ __forceinline__ float half_bits(uint16_t v, int half_f16) {
  return half_f16 ? f16_bits_to_f32(v) : bf16_bits_to_f32(v);
}

// Grid (d_ff / 8, k + S), 256 threads.  MSW: slabs per wave (the reduction
// split in four); MPL: router logits per lane in the selection (E <= 64*MPL).
template <int QB, int MSW, int MPL>
__global__ __launch_bounds__(256) void t1_gateup_kernel(T1Args a) {
  __shared__ __align__(16) uint16_t xs[kT1MaxD];  // fp16 staging row of x (zero past D to whole slabs)
  __shared__ int8_t s_xsh;
  __shared__ int32_t s_idx[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float part[kGUWaves][16];

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;
  // one XCD per range of consecutive (slot, column block) pairs: the 8 column
  // blocks whose scales and biases share a cache line share an L2
  const int nx = gridDim.x;
  const int item = xcd_contiguous(blockIdx.y * nx + blockIdx.x, nx * gridDim.y);
  const int slot = item / nx, cb = item % nx;
  const int D = a.D, F = a.F, nslab = (D + kSlab - 1) / kSlab;

  // the token's experts (wave 0) and the fp16 staging row of x (wave 1)
  if (wave == 0) {
    select_token<MPL>(0, a.partials, a.n_chunks, a.bias, 1, a.E, a.K, a.renorm, s_idx, s_w, nullptr, D, nullptr,
                      nullptr, false, XgOut{nullptr, 0, 0}, nullptr);
  } else if (wave == 1) {
    row_to_f16(a.x, D, xs, &s_xsh, a.x_f16 != 0);
  } else {
    for (int q = (tid - 2 * kWave) * 8 + D; q < nslab * kSlab; q += 2 * kWave * 8)
      *reinterpret_cast<uint4 *>(&xs[q]) = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid < a.K) {
    a.idx[tid] = s_idx[tid];
    a.wt[tid] = s_w[tid];
  }
  const int e = slot < a.K ? s_idx[slot] : a.E + (slot - a.K);

  // this lane's weight row: gate column (lr < 8) or up column (lr >= 8) of cb*8 + lr%8
  const bool up = lr >= 8;
  const int col = cb * 8 + (lr & 7);
  const int nre = a.fused ? 2 * F : F;
  const int rin = (a.fused && up ? F : 0) + col;
  const bool second = !a.fused && up;
  const int KW = D * QB / 32, G = D / a.gsize;
  const uint32_t *wrow = (second ? a.wu : a.wg) + (int64_t(e) * nre + rin) * KW;
  const uint16_t *sp = (second ? a.su : a.sg) + int64_t(e) * G * nre + rin;
  const uint16_t *bp = (second ? a.bu : a.bg) + int64_t(e) * G * nre + rin;
  const int nsw = (nslab + kGUWaves - 1) / kGUWaves;
  const int s0 = wave * nsw, ns = min(nsw, nslab - s0);  // this wave's slabs (ns may be <= 0)

  uint4 wq[MSW][QB / 4];
  uint16_t sr[MSW], br[MSW];
#pragma unroll
  for (int s = 0; s < MSW; ++s)
    load_row_slab<QB>(wrow, sp, bp, nre, D, a.gsize, min(s0 + s, nslab - 1), lg, s < ns, wq[s], sr[s], br[s]);

  uint32_t magic = QB == 8 ? 0x64646464u : 0x64006400u;
  asm volatile("" : "+v"(magic));
  float tot = 0.f;
#pragma unroll
  for (int s = 0; s < MSW; ++s) {
    if (s < ns) {
      float qx, sx;
      slab_dot<QB>(wq[s], xs + (s0 + s) * kSlab + lg * 32, magic, qx, sx);
      tot = __builtin_fmaf(half_bits(sr[s], a.half_f16), qx, __builtin_fmaf(half_bits(br[s], a.half_f16), sx, tot));
    }
  }
  // the row's four lanes lg, then the waves' partial sums in LDS (true values)
  tot += __shfl_xor(tot, 16, kWave);
  tot += __shfl_xor(tot, 32, kWave);
  if (lane < 16) part[wave][lane] = ns > 0 ? tot * pow2(int(s_xsh)) : 0.f;
  __syncthreads();
  if (wave == 0) {
    float hv = 0.f;
    if (lane < 8) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < kGUWaves; ++w) {
        g += part[w][lane];
        u += part[w][8 + lane];
      }
      hv = glu(g, u, a.round_ops, a.geglu != 0);
      a.h[int64_t(slot) * F + cb * 8 + lane] = hv;
    }
    float m = fabsf(hv);
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    m = fmaxf(m, __shfl_xor(m, 4, kWave));
    if (lane == 0) a.hmax[slot * (F / 8) + cb] = m;
  }
}

// Grid d_model / 16, 512 threads.  MS: slabs of d_ff held per wave.
template <int QB, int MS>
__global__ __launch_bounds__(512) void t1_down_combine_kernel(T1Args a) {
  extern __shared__ __align__(16) uint16_t hs[];  // [k + S][FR] fp16 h rows (staging order, zero to whole slabs)
  __shared__ uint32_t rmax_bits[kMaxTopK + kMaxShared];
  __shared__ float part[kDNWaves][16];

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int D = a.D, F = a.F, nslab = (F + kSlab - 1) / kSlab, FR = nslab * kSlab;
  const int R = a.K + a.S;
  // consecutive 16-column blocks (whose scales share cache lines) on one XCD
  const int c0 = xcd_contiguous(blockIdx.x, gridDim.x) * 16;

  // weights of this wave's first slot, issued before the h rows are staged
  auto slot_expert = [&](int j) { return j < a.K ? a.idx[j] : a.E + (j - a.K); };
  const int G = F / a.gsize, KW = F * QB / 32;
  uint4 wq[MS][QB / 4];
  uint16_t sr[MS], br[MS];
  auto load_slot = [&](int j) {
    const int e = slot_expert(j);
    const uint32_t *wrow = a.wd + (int64_t(e) * D + c0 + lr) * KW;
    const uint16_t *sp = a.sd + int64_t(e) * G * D + c0 + lr, *bp = a.bd + int64_t(e) * G * D + c0 + lr;
#pragma unroll
    for (int s = 0; s < MS; ++s)
      load_row_slab<QB>(wrow, sp, bp, D, F, a.gsize, min(s, nslab - 1), lg, s < nslab, wq[s], sr[s], br[s]);
  };
  if (wave < R) load_slot(wave);

  // h rows as fp16, one exponent per row (from the gate/up blocks' maxima):
  // the h pieces of this thread and the maxima are loaded together, the row
  // maxima formed with LDS atomics on the (nonnegative) float bits.
  const int P = F / 8;  // 8-element pieces per row
  float4 hv[kT1HPieces][2];
#pragma unroll
  for (int i = 0; i < kT1HPieces; ++i) {
    const int q = min(tid + i * 512, R * P - 1);
    const float4 *p = reinterpret_cast<const float4 *>(a.h + int64_t(q / P) * F + (q % P) * 8);
    hv[i][0] = p[0];
    hv[i][1] = p[1];
  }
  // (the block maxima [R][F/8] are indexed like the pieces)
  float bm[kT1HPieces];
#pragma unroll
  for (int i = 0; i < kT1HPieces; ++i) bm[i] = a.hmax[min(tid + i * 512, R * P - 1)];
  if (tid < R) rmax_bits[tid] = 0u;
  for (int q = tid; q < R * (FR - F) / 8; q += blockDim.x) {
    const int nz = (FR - F) / 8;
    *reinterpret_cast<uint4 *>(&hs[(q / nz) * FR + F + (q % nz) * 8]) = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kT1HPieces; ++i)
    if (tid + i * 512 < R * P) atomicMax(&rmax_bits[(tid + i * 512) / P], __float_as_uint(bm[i]));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kT1HPieces; ++i) {
    const int q = tid + i * 512;
    if (q < R * P) {
      const int r = q / P;
      const float m = pow2(-f16_shift(__uint_as_float(rmax_bits[r])));
      const float vv[8] = {hv[i][0].x, hv[i][0].y, hv[i][0].z, hv[i][0].w,
                           hv[i][1].x, hv[i][1].y, hv[i][1].z, hv[i][1].w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = __builtin_bit_cast(uint32_t, h2{(_Float16)(vv[k] * m), (_Float16)(vv[k + 4] * m)});
      // staging order e0,e4,e1,e5,e2,e6,e3,e7
      *reinterpret_cast<uint4 *>(&hs[r * FR + (q % P) * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  __syncthreads();

  uint32_t magic = QB == 8 ? 0x64646464u : 0x64006400u;
  asm volatile("" : "+v"(magic));
  float ysum = 0.f;  // output column c0 + lr, this lane's quarter lg of every slab
  for (int j = wave; j < R; j += kDNWaves) {
    if (j != wave) load_slot(j);
    float tot = 0.f;
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      if (s < nslab) {
        float qx, sx;
        slab_dot<QB>(wq[s], hs + j * FR + s * kSlab + lg * 32, magic, qx, sx);
        tot = __builtin_fmaf(half_bits(sr[s], a.half_f16), qx, __builtin_fmaf(half_bits(br[s], a.half_f16), sx, tot));
      }
    }
    const float c = j < a.K ? a.wt[j] : 1.0f;
    ysum += c * (tot * pow2(f16_shift(__uint_as_float(rmax_bits[j]))));
  }
  ysum += __shfl_xor(ysum, 16, kWave);
  ysum += __shfl_xor(ysum, 32, kWave);
  if (lane < 16) part[wave][lane] = ysum;
  __syncthreads();
  if (tid < 16) {
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kDNWaves; ++w) y += part[w][tid];
    if (a.out_dtype == MOE_DT_F32) static_cast<float *>(a.y)[c0 + tid] = y;
    else if (a.out_dtype == MOE_DT_BF16) static_cast<uint16_t *>(a.y)[c0 + tid] = uint16_t(f32_to_bf16_bits(y));
    else static_cast<uint16_t *>(a.y)[c0 + tid] = uint16_t(f32_to_f16_bits(y));
  }
}

template <int QB>
void launch_t1_qb(const T1Args &a, hipStream_t s) {
  const int nslab_d = (a.D + kSlab - 1) / kSlab, nsw = (nslab_d + kGUWaves - 1) / kGUWaves;
  const dim3 g1(a.F / 8, a.K + a.S);
  auto gu = [&](auto msw) {
    constexpr int MSW = decltype(msw)::value;
    if (a.E <= 64) launch((t1_gateup_kernel<QB, MSW, 1>), g1, dim3(256), 0, s, a);
    else if (a.E <= 128) launch((t1_gateup_kernel<QB, MSW, 2>), g1, dim3(256), 0, s, a);
    else if (a.E <= 256) launch((t1_gateup_kernel<QB, MSW, 4>), g1, dim3(256), 0, s, a);
    else if (a.E <= 512) launch((t1_gateup_kernel<QB, MSW, 8>), g1, dim3(256), 0, s, a);
    else launch((t1_gateup_kernel<QB, MSW, 16>), g1, dim3(256), 0, s, a);
  };
  if (nsw <= 4) gu(std::integral_constant<int, 4>{});
  else gu(std::integral_constant<int, 8>{});
}

template <int QB>
void launch_t1_down(const T1Args &a, hipStream_t s) {
  const int nslab = (a.F + kSlab - 1) / kSlab;
  const size_t lds = size_t(a.K + a.S) * nslab * kSlab * sizeof(uint16_t);
  const dim3 g2(a.D / 16);
  if (QB == 8 || nslab <= 8) launch((t1_down_combine_kernel<QB, 8>), g2, dim3(512), lds, s, a);
  else launch((t1_down_combine_kernel<QB, QB == 8 ? 8 : 16>), g2, dim3(512), lds, s, a);
}

}  // namespace

bool t1_fused_applies(const moe_layer_desc *d, int32_t T) {
  const int64_t R = int64_t(d->top_k) + d->n_shared;
  const int64_t fr = (d->d_ff + kSlab - 1) / kSlab * kSlab;
  // 8-bit codes of a d_ff above 1024 would not fit the down waves' registers
  const int max_f = d->w_format == MOE_WF_AFFINE_Q8 ? kT1MaxF / 2 : kT1MaxF;
  // (the h block maxima, [k+S][d_ff/8], live in the expert-output section,
  // which holds at least [k+S][d_model] fp32 at one token)
  return T == 1 && use_mfma(d) && affine(d) && d->d_model <= kT1MaxD && d->d_ff <= max_f &&
         R * fr <= kT1MaxHStage && d->d_ff / 8 <= d->d_model;
}

void launch_t1_layer(const moe_layer_desc *d, const void *x, const moe_weights *w, const float *partials,
                     int n_chunks, int32_t *idx, float *wt, float *h, float *hmax, void *y, int32_t out_dtype,
                     void *stream, StageMarker *mk) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_proj &pg = d->gate_up_fused ? w->gate_up : w->gate;
  T1Args a{partials, n_chunks, w->router_bias, d->n_experts, d->top_k, d->n_shared, d->renormalize,
           static_cast<const uint16_t *>(x), d->act_dtype == MOE_DT_F16, d->d_model, d->d_ff, d->gate_up_fused,
           glu_round_mode(d), d->activation == MOE_ACT_GEGLU, d->group_size, d->act_dtype == MOE_DT_F16,
           static_cast<const uint32_t *>(pg.w), static_cast<const uint16_t *>(pg.scales),
           static_cast<const uint16_t *>(pg.biases), static_cast<const uint32_t *>(w->up.w),
           static_cast<const uint16_t *>(w->up.scales), static_cast<const uint16_t *>(w->up.biases),
           static_cast<const uint32_t *>(w->down.w), static_cast<const uint16_t *>(w->down.scales),
           static_cast<const uint16_t *>(w->down.biases), idx, wt, h, hmax, y, out_dtype};
  if (d->w_format == MOE_WF_AFFINE_Q8) launch_t1_qb<8>(a, s);
  else launch_t1_qb<4>(a, s);
  if (mk) mk->mark("select_gateup");
  if (d->w_format == MOE_WF_AFFINE_Q8) launch_t1_down<8>(a, s);
  else launch_t1_down<4>(a, s);
  if (mk) mk->mark("down_combine");
}

}  // namespace moe
