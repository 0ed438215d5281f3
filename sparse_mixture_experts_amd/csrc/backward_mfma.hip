// backward_mfma.hip -- the backward pass of 16-bit layers on the matrix cores.
//
// "SwitchGLU: grouped-expert Metal kernels" (ml-explore/mlx-lm #2044),
// section "What": the grouped expert kernels carry a custom VJP.  The pass is
// the chain of contractions of the fp32 vector-unit kernels, over the same
// grouping of sorted rows by expert (the forward's plan tiles):
//   g | u = x Wgu^T     the forward's grouped GEMM, run as a plain projection
//                       on a gathered copy of the sorted rows' x
//   v     = dy Wd       transposed use of the down weights
//   dw, dg | du         per row, from g, u, v and the slot weight (GLU derivative)
//   dx_r  = [dg|du] Wgu transposed use of the gate/up weights
//
// Transposed use.  The stored matrices keep the forward's reduction dimension
// contiguous (codes packed and quantised in groups along a row), so v and
// dx_r reduce over the stored row index.  A workgroup owns one plan tile (up
// to 16*RB rows of one expert), 128 output columns (stored columns) and a
// range of the reduction.  Per slab of 64 reduction rows the 256 threads load
// the codes, dequantise them in fp32 (s*q + b), round to bf16 and write each
// pair of consecutive reduction rows of one column as one dword, so LDS holds
// [32 row pairs][128 columns]; an MFMA operand (8 consecutive reduction rows
// of one column) is then four dword reads.  The activations (dy gathered by
// token and rounded to bf16, or the bf16 dg|du rows) are staged as
// [rows][64].  v_mfma_f32_16x16x32_bf16 takes 16 weight columns as operand A
// and 16 rows as operand B; fp32 accumulation.  bf16 operands keep every
// value in range without exponent bookkeeping (dy is arbitrary fp32).
//
// Small row counts split the reduction over several workgroups; each split
// writes its own partial sums and the consumers (the GLU kernel for v, the
// per-token sum for dx) add them in split order, so results do not depend on
// scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "f16_stage.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTN = 128;              // output columns per workgroup
constexpr int kTK = 64;               // reduction rows per slab
constexpr int kPairs = kTK / 2;       // LDS row pairs per slab
constexpr int kPairStride = kTN + 4;  // dwords per LDS pair row: the four lane groups of a read hit different banks
constexpr int kARow = kTK + 8;        // bf16 elements per LDS activation row

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- gathered x ------------------------------------------------------------
// Sorted row r of x (token row_map[r], or (r - N) % T for shared rows) in the
// activation format of the grouped GEMM: affine layers fp16 with the row's
// exponent repeated for each 128-column block; dense layers a plain copy.
// One wave per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *x, const int32_t *row_map, int T, int N,
                                                          int R, int D, int nblk, int aff, int x_f16, uint16_t *xs,
                                                          int8_t *xsh) {
  const int r = blockIdx.x * (256 / kWave) + int(threadIdx.x) / kWave;
  if (r >= R) return;  // whole waves
  const int tok = r < N ? row_map[r] : (r - N) % T;
  const uint16_t *src = x + int64_t(tok) * D;
  uint16_t *dst = xs + int64_t(r) * D;
  if (aff) {
    row_to_f16(src, D, dst, xsh + int64_t(r) * nblk, x_f16 != 0);
    if (lane_id() == 0) {
      const int8_t e = xsh[int64_t(r) * nblk];  // written by this lane just above
      for (int b = 1; b < nblk; ++b) xsh[int64_t(r) * nblk + b] = e;
    }
  } else {
    for (int p = lane_id(); p < D / 8; p += kWave)
      reinterpret_cast<uint4 *>(dst)[p] = reinterpret_cast<const uint4 *>(src)[p];
  }
}

// ---- transposed grouped GEMM -------------------------------------------------
struct TArgs {
  const void *act;        // ASRC 0: fp32 [T][K] read through the rows' tokens; 1: bf16 [R][K] sorted rows
  const int32_t *row_map;
  int T, N;               // tokens, routed rows
  int K;                  // reduction length
  int n_cols;             // output columns = stored row length of the weights
  int k_second;           // reduction rows k >= k_second come from matrix 1 (row k - k_second)
  const void *w[2];       // codes [E+S][nre][n_cols*bits/32] words, or 16-bit [E+S][nre][n_cols]
  const uint16_t *sc[2], *bi[2];  // affine: [E+S][n_cols/group][nre]
  int nre[2];             // stored rows of one expert's matrix
  int group;
  int half_f16;           // scales/biases or dense weights are fp16 (else bf16)
  const int32_t *counters;  // [1] = plan tiles
  const PlanItem *tiles;
  float *out;             // [ksplit][R][n_cols]
  int64_t split_stride;   // elements between two splits' partial sums
  int ksplit;
};

// QB: 4 or 8 (affine codes) or 16 (dense 16-bit weights).  RB: 16-row blocks
// per tile.  ASRC: activation source (see TArgs::act).  HF: scales/biases or
// dense weights are fp16 (else bf16).
template <int QB, int RB, int ASRC, bool HF>
__global__ __launch_bounds__(kThreads) void tgemm_kernel(TArgs a) {
  constexpr bool AFF = QB != 16;
  constexpr int VPW = 32 / QB;         // values per 32-bit word (8, 4, 2)
  constexpr int WPR = kTN / VPW;       // words per slab row and column block (16, 32, 64)
  constexpr int PPP = kThreads / WPR;  // row pairs per staging pass (16, 8, 4)
  constexpr int NPASS = kPairs / PPP;  // staging passes (2, 4, 8)
  constexpr int PPR = kTK / 8;         // 8-element activation pieces per row (8)
  constexpr int RPP = kThreads / PPR;  // activation rows per staging pass (32)
  constexpr int APASS = (RB * 16 + RPP - 1) / RPP;
  static_assert(kThreads % WPR == 0 && kPairs % PPP == 0, "weight staging covers the slab");
  __shared__ uint32_t bt[2][kPairs * kPairStride];
  __shared__ uint16_t as[2][RB * 16 * kARow];

  // XCD-aware order: consecutive linear ids go to the 8 XCDs in turn; the
  // work items (tile, column block, split) are cut into 8 contiguous ranges,
  // one per XCD, so the column blocks of a tile share an L2.
  const int nbx = gridDim.x;
  const int total = nbx * gridDim.y;
  const int work = a.counters[1] * nbx;
  const int lin = blockIdx.y * nbx + blockIdx.x;
  const int per = (work + 7) / 8;
  int item = lin;
  if (8 * per <= total) {
    const int slot = lin / 8;
    if (slot >= per) return;
    item = (lin % 8) * per + slot;
  }
  if (item >= work) return;
  const int ncb = (a.n_cols + kTN - 1) / kTN;
  const int tile_id = item / nbx, bx = item % nbx;
  const int cb = bx % ncb, z = bx / ncb;
  const PlanItem tile = a.tiles[tile_id];
  const int n0 = cb * kTN;
  const int ks = a.K / a.ksplit;  // whole slabs (the host picks the split)
  const int k_begin = z * ks, nsl = ks / kTK;

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;

  // Weight staging role: word column wc of the block, row pairs pr + i*PPP
  // of every slab.  Per matrix, this thread's word (and scale pair) of row 0
  // of the slab; a slab adds its first row, a pass 2*PPP rows.
  const int wc = tid % WPR, pr = tid / WPR;
  const int wpr_row = a.n_cols / VPW;                 // words per stored row
  const int wcol = min(n0 / VPW + wc, wpr_row - 1);   // clamped (columns past n_cols are never stored)
  const int ngrp = AFF ? a.n_cols / a.group : 1;
  const int grp = AFF ? wcol * VPW / a.group : 0;
  const uint32_t *wbase[2];
  const uint32_t *sbase[2], *bbase[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    wbase[m] = static_cast<const uint32_t *>(a.w[m]) + (int64_t(tile.expert) * a.nre[m] + 2 * pr) * wpr_row + wcol;
    if constexpr (AFF) {
      const int64_t si = (int64_t(tile.expert) * ngrp + grp) * a.nre[m] + 2 * pr;
      sbase[m] = reinterpret_cast<const uint32_t *>(a.sc[m] + si);  // (row, row + 1) scale pair
      bbase[m] = reinterpret_cast<const uint32_t *>(a.bi[m] + si);
    }
  }
  const int pass_w = 2 * PPP * wpr_row;

  uint32_t wr[NPASS][2];
  uint32_t sr[NPASS], br[NPASS];
  auto load_w = [&](int slab) {
    const int k = k_begin + slab * kTK;  // the slab lies in one matrix (k_second is a multiple of kTK)
    const int m = k >= a.k_second ? 1 : 0;
    const int row = k - (m ? a.k_second : 0);
    const uint32_t *wp = (m ? wbase[1] : wbase[0]) + row * wpr_row;
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      wr[i][0] = wp[i * pass_w];
      wr[i][1] = wp[i * pass_w + wpr_row];
    }
    if constexpr (AFF) {
      const uint32_t *sp = (m ? sbase[1] : sbase[0]) + row / 2;
      const uint32_t *bp = (m ? bbase[1] : bbase[0]) + row / 2;
#pragma unroll
      for (int i = 0; i < NPASS; ++i) {
        sr[i] = sp[i * PPP];
        br[i] = bp[i * PPP];
      }
    }
  };
  auto write_w = [&](uint32_t *dst) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      uint32_t o[VPW];
      if constexpr (AFF) {
        const float s0 = HF ? f16_lo(sr[i]) : bf16_lo(sr[i]), s1 = HF ? f16_hi(sr[i]) : bf16_hi(sr[i]);
        const float b0 = HF ? f16_lo(br[i]) : bf16_lo(br[i]), b1 = HF ? f16_hi(br[i]) : bf16_hi(br[i]);
        float q0[VPW], q1[VPW];
        if constexpr (QB == 4) {
          // even codes in the low nibbles of the four bytes, odd codes in the
          // high ones: eight byte-to-float conversions per word
          uint32_t e0 = wr[i][0] & 0x0f0f0f0fu, o0 = (wr[i][0] >> 4) & 0x0f0f0f0fu;
          uint32_t e1 = wr[i][1] & 0x0f0f0f0fu, o1 = (wr[i][1] >> 4) & 0x0f0f0f0fu;
          asm volatile("" : "+v"(e0), "+v"(o0), "+v"(e1), "+v"(o1));  // keep whole-byte conversions
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            q0[2 * b] = float((e0 >> (8 * b)) & 0xffu);
            q0[2 * b + 1] = float((o0 >> (8 * b)) & 0xffu);
            q1[2 * b] = float((e1 >> (8 * b)) & 0xffu);
            q1[2 * b + 1] = float((o1 >> (8 * b)) & 0xffu);
          }
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            q0[b] = float((wr[i][0] >> (8 * b)) & 0xffu);
            q1[b] = float((wr[i][1] >> (8 * b)) & 0xffu);
          }
        }
#pragma unroll
        for (int j = 0; j < VPW; ++j) o[j] = pack_bf16(__builtin_fmaf(s0, q0[j], b0), __builtin_fmaf(s1, q1[j], b1));
      } else if constexpr (HF) {
        o[0] = pack_bf16(f16_lo(wr[i][0]), f16_lo(wr[i][1]));
        o[1] = pack_bf16(f16_hi(wr[i][0]), f16_hi(wr[i][1]));
      } else {
        o[0] = (wr[i][0] & 0xffffu) | (wr[i][1] << 16);
        o[1] = (wr[i][0] >> 16) | (wr[i][1] & 0xffff0000u);
      }
      uint32_t *d = dst + (pr + i * PPP) * kPairStride + wc * VPW;
      if constexpr (VPW == 8) {
        reinterpret_cast<uint4 *>(d)[0] = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4 *>(d)[1] = make_uint4(o[4], o[5], o[6], o[7]);
      } else if constexpr (VPW == 4) {
        *reinterpret_cast<uint4 *>(d) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        *reinterpret_cast<uint2 *>(d) = make_uint2(o[0], o[1]);
      }
    }
  };

  // activation staging role: piece pc of rows rr + i*RPP
  const int pc = tid % PPR, rr = tid / PPR;
  int64_t aoff[APASS];
  bool aok[APASS];
#pragma unroll
  for (int i = 0; i < APASS; ++i) {
    const int m = rr + i * RPP;
    aok[i] = m < tile.rows && m < RB * 16;
    const int q = tile.row0 + (aok[i] ? m : 0);
    int src = q;
    if constexpr (ASRC == 0) src = q < a.N ? a.row_map[q] : (q - a.N) % a.T;
    aoff[i] = int64_t(src) * a.K + pc * 8;
  }
  float4 af[APASS][2];
  uint4 ab[APASS];
  auto load_a = [&](int slab) {
    const int k = k_begin + slab * kTK;
#pragma unroll
    for (int i = 0; i < APASS; ++i) {
      if constexpr (ASRC == 0) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.act) + aoff[i] + k);
        af[i][0] = p[0];
        af[i][1] = p[1];
      } else {
        ab[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + aoff[i] + k);
      }
    }
  };
  auto write_a = [&](uint16_t *dst) {
#pragma unroll
    for (int i = 0; i < APASS; ++i) {
      const int m = rr + i * RPP;
      if (m < RB * 16) {
        uint4 v;
        if constexpr (ASRC == 0) {
          v = make_uint4(pack_bf16(af[i][0].x, af[i][0].y), pack_bf16(af[i][0].z, af[i][0].w),
                         pack_bf16(af[i][1].x, af[i][1].y), pack_bf16(af[i][1].z, af[i][1].w));
        } else {
          v = ab[i];
        }
        if (!aok[i]) v = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4 *>(dst + m * kARow + pc * 8) = v;
      }
    }
  };

  f32x4 acc[2][RB];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[ct][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int cw = wave * 32 + lr;  // this lane's operand-A column (plus 16 for the second tile)
  auto compute = [&](const uint32_t *bsl, const uint16_t *asl) {
#pragma unroll
    for (int j = 0; j < kTK / 32; ++j) {
      bf16x8 wa[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint32_t *p = bsl + (16 * j + 4 * lg) * kPairStride + cw + 16 * ct;
        const uint4 v = make_uint4(p[0], p[kPairStride], p[2 * kPairStride], p[3 * kPairStride]);
        wa[ct] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb * 16 < tile.rows) {  // uniform
          const uint4 v = *reinterpret_cast<const uint4 *>(asl + (rb * 16 + lr) * kARow + 32 * j + 8 * lg);
          const bf16x8 xb = __builtin_bit_cast(bf16x8, v);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            acc[ct][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ct], xb, acc[ct][rb], 0, 0, 0);
        }
      }
    }
  };

  // Double buffer: slab i is multiplied from LDS while slab i+1 waits in
  // registers to be written to the other buffer and slab i+2 is in flight.
  load_w(0);
  load_a(0);
  write_w(bt[0]);
  write_a(as[0]);
  if (nsl > 1) {
    load_w(1);
    load_a(1);
  }
  __syncthreads();
  for (int i = 0; i < nsl; ++i) {
    compute(bt[i & 1], as[i & 1]);
    if (i + 1 < nsl) {
      write_w(bt[(i + 1) & 1]);
      write_a(as[(i + 1) & 1]);
    }
    if (i + 2 < nsl) {
      load_w(i + 2);
      load_a(i + 2);
    }
    __syncthreads();
  }

  // lane holds outputs n = column + 4*lg + e (e = 0..3) of tile row rb*16 + lr
  float *out = a.out + int64_t(z) * a.split_stride;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = rb * 16 + lr;
    if (m >= tile.rows) continue;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = n0 + wave * 32 + 16 * ct + 4 * lg;
      if (n < a.n_cols)
        *reinterpret_cast<float4 *>(out + int64_t(tile.row0 + m) * a.n_cols + n) =
            make_float4(acc[ct][rb][0], acc[ct][rb][1], acc[ct][rb][2], acc[ct][rb][3]);
    }
  }
}

// ---- GLU backward per sorted row ---------------------------------------------
// dw_r = h . v and dg = c v u a'(g), du = c v a(g), written as bf16 [R][2F]
// (dg then du), with v the sum of the split partials.
struct GluArgs {
  const float *g, *u;
  int gu_stride;
  const float *v;
  int vsplit;
  int64_t v_split_stride;
  const float *topk_w;
  const int32_t *order;
  int N, F, geglu;
  float *dw;
  uint16_t *dgu;
};
__global__ __launch_bounds__(256) void glu_bf16_kernel(GluArgs a) {
  __shared__ float part[256 / kWave];
  const int r = blockIdx.x;
  const float c = r < a.N ? a.topk_w[a.order[r]] : 1.0f;
  float dwp = 0.f;
  for (int f = threadIdx.x; f < a.F; f += 256) {
    const float g = a.g[int64_t(r) * a.gu_stride + f], u = a.u[int64_t(r) * a.gu_stride + f];
    float v = 0.f;
    for (int z = 0; z < a.vsplit; ++z) v += a.v[z * a.v_split_stride + int64_t(r) * a.F + f];
    float act, dact;
    gate_act_grad(g, a.geglu != 0, act, dact);
    dwp = __builtin_fmaf(act * u, v, dwp);
    const float dh = c * v;
    a.dgu[int64_t(r) * 2 * a.F + f] = uint16_t(f32_to_bf16_bits(dh * u * dact));
    a.dgu[int64_t(r) * 2 * a.F + a.F + f] = uint16_t(f32_to_bf16_bits(dh * act));
  }
  dwp = wave_sum(dwp);
  if (lane_id() == 0) part[threadIdx.x / kWave] = dwp;
  __syncthreads();
  if (threadIdx.x == 0) a.dw[r] = (part[0] + part[1]) + (part[2] + part[3]);
}

template <int QB, int RB, bool HF>
void launch_t_src(const TArgs &t, int asrc, int64_t max_tiles, hipStream_t s) {
  const dim3 grid(unsigned(((t.n_cols + kTN - 1) / kTN) * t.ksplit), unsigned(max_tiles));
  if (asrc == 0) hipLaunchKernelGGL((tgemm_kernel<QB, RB, 0, HF>), grid, dim3(kThreads), 0, s, t);
  else hipLaunchKernelGGL((tgemm_kernel<QB, RB, 1, HF>), grid, dim3(kThreads), 0, s, t);
}
template <int QB, int RB>
void launch_t_hf(const TArgs &t, int asrc, int64_t max_tiles, hipStream_t s) {
  if (t.half_f16) launch_t_src<QB, RB, true>(t, asrc, max_tiles, s);
  else launch_t_src<QB, RB, false>(t, asrc, max_tiles, s);
}
template <int RB>
void launch_t_rb(const TArgs &t, int qb, int asrc, int64_t max_tiles, hipStream_t s) {
  if (qb == 4) launch_t_hf<4, RB>(t, asrc, max_tiles, s);
  else if (qb == 8) launch_t_hf<8, RB>(t, asrc, max_tiles, s);
  else launch_t_hf<16, RB>(t, asrc, max_tiles, s);
}
void launch_t(const TArgs &t, int qb, int tile_rows, int asrc, int64_t max_tiles, hipStream_t s) {
  if (tile_rows == 16) launch_t_rb<1>(t, qb, asrc, max_tiles, s);
  else launch_t_rb<4>(t, qb, asrc, max_tiles, s);
}

}  // namespace

BwdSplits backward_splits(const moe_layer_desc *d, int32_t T) {
  if (!use_mfma(d)) return {1, 1};
  const int64_t R = int64_t(T) * d->top_k + int64_t(d->n_shared) * T;
  // rough count of plan tiles: one per touched expert for small groups, one
  // per 64 rows for large ones
  const int64_t tiles = std::max<int64_t>(std::min<int64_t>(R, d->n_experts + d->n_shared), R / 64);
  auto pick = [&](int n_cols, int K) {
    const int64_t blocks = tiles * ((n_cols + kTN - 1) / kTN);
    int s = 1;
    while (blocks * s < 1024 && s < 8 && K % (2 * s * 2 * kTK) == 0) s *= 2;  // at least two slabs per split
    return s;
  };
  return {pick(d->d_ff, d->d_model), pick(d->d_model, 2 * d->d_ff)};
}

void launch_backward_mfma(const moe_layer_desc *d, int32_t T, const void *x, const moe_weights *w, const float *dy,
                          const float *topk_w, const int32_t *order, const int32_t *row_map,
                          const int32_t *counters, const PlanItem *tiles, int64_t max_tiles, const BwdScratch &sc,
                          void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_model, F = d->d_ff, K = d->top_k;
  const int N = T * K, R = N + d->n_shared * T;
  const bool aff = affine(d);
  const int f16 = d->act_dtype == MOE_DT_F16;
  const int qb = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : aff ? 4 : 16;
  const int tr = plan_tile_rows(d, T);
  const BwdSplits sp = backward_splits(d, T);
  const int nblk = (D + kHBlock - 1) / kHBlock;
  const bool fused = d->gate_up_fused;

  // 1. g | u on the forward's grouped GEMM, from the sorted rows of x
  hipLaunchKernelGGL(gather_rows_kernel, dim3((R + 3) / 4), dim3(256), 0, s, static_cast<const uint16_t *>(x),
                     row_map, T, N, R, D, nblk, int(aff), f16, static_cast<uint16_t *>(sc.xs), sc.xsh);
  if (fused) {
    launch_projection_mfma(d, T, sc.xs, sc.xsh, D, 2 * F, w->gate_up, counters, tiles, max_tiles, sc.gu, stream);
  } else {
    launch_projection_mfma(d, T, sc.xs, sc.xsh, D, F, w->gate, counters, tiles, max_tiles, sc.gu, stream);
    launch_projection_mfma(d, T, sc.xs, sc.xsh, D, F, w->up, counters, tiles, max_tiles, sc.gu + int64_t(R) * F,
                           stream);
  }

  // 2. v = dy Wd (down weights [E+S][D][F]: reduction over d, columns f)
  const moe_proj &dn = w->down;
  TArgs tv{dy, row_map, T, N, D, F, D,
           {dn.w, dn.w}, {static_cast<const uint16_t *>(dn.scales), static_cast<const uint16_t *>(dn.scales)},
           {static_cast<const uint16_t *>(dn.biases), static_cast<const uint16_t *>(dn.biases)}, {D, D},
           d->group_size, f16, counters, tiles, sc.v, int64_t(R) * F, sp.v};
  launch_t(tv, qb, tr, 0, max_tiles, s);

  // 3. dw and dg | du per row
  GluArgs ga{sc.gu, fused ? sc.gu + F : sc.gu + int64_t(R) * F, fused ? 2 * F : F, sc.v, sp.v, int64_t(R) * F,
             topk_w, order, N, F, d->activation == MOE_ACT_GEGLU, sc.dw, sc.dgu};
  hipLaunchKernelGGL(glu_bf16_kernel, dim3(R), dim3(256), 0, s, ga);

  // 4. dx_r = [dg | du] Wgu (gate rows then up rows: reduction over 2F, columns d)
  const moe_proj &pg = fused ? w->gate_up : w->gate, &pu = fused ? w->gate_up : w->up;
  TArgs tx{sc.dgu, row_map, T, N, 2 * F, D, fused ? 2 * F : F,
           {pg.w, pu.w}, {static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pu.scales)},
           {static_cast<const uint16_t *>(pg.biases), static_cast<const uint16_t *>(pu.biases)},
           {fused ? 2 * F : F, fused ? 2 * F : F}, d->group_size, f16, counters, tiles, sc.dxr, int64_t(R) * D,
           sp.dx};
  launch_t(tx, qb, tr, 1, max_tiles, s);
}

}  // namespace moe
