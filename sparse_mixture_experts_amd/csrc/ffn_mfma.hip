// ffn_mfma.hip -- grouped expert GEMMs on the bf16 matrix cores (MFMA).
//
// The sorted-row route of DS4Server issue #112 ("Current upstream route",
// "Kernel contract"): workgroups own a tile of one expert's sorted rows; the
// gate/up kernel reads token rows in place through row_map and writes
// silu(gate) * up directly (per-op activation-dtype rounding when asked); the
// down kernel runs on the already sorted, contiguous h rows.  Grouping rows by
// expert means each expert's weights are read and dequantised once per tile
// ("SwitchGLU: grouped-expert Metal kernels", section "What").
//
// gfx950 mapping.  One v_mfma_f32_16x16x32_bf16 multiplies a 16x32 weight
// block (operand A: 16 weight rows n) by a 32x16 activation block (operand B:
// 16 token rows m).  A lane holds row/column l%16 and the 8 reduction elements
// 8*(l/16)..+8 of its operand; its 4 results are rows n = 4*(l/16)+i of
// column m = l%16, i.e. 4 consecutive outputs of one token row, which makes
// the stores contiguous.
//
// Weight operands come straight from global memory into registers (every
// weight element is used by exactly one lane): for affine 4-bit weights a lane
// reads 2 words = 16 codes of one quantisation group per step and turns each
// word into 8 bf16 values 128+q with one shift and one and-or per pair (the
// bf16 with exponent 2^7 and the code as its low mantissa bits is exactly
// 128+q).  The pairs come out as (q_j, q_{j+4}), so the activations are
// staged in LDS with the same order inside every 8-element block.  Since
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k
// per 64-element group, two MFMAs give D = sum x (128+q) for the group and
// the fp32 epilogue of the group adds s*D + (b - 128 s)*X with X the group sum
// of the activations (computed once per staged row).  Dense bf16 weights go
// to the MFMA unchanged.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kKS = 256;       // reduction elements staged in LDS per slab
constexpr int kPad = 8;        // bf16 padding per LDS row (bank spread)
constexpr int kLdsRow = kKS + kPad;
constexpr int kGroupsPerSlab = kKS / kGroup;

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 codes of a word -> 8 bf16 (128 + q) in the order q0,q4,q1,q5,q2,q6,q3,q7.
__device__ __forceinline__ bf16x8 q4_word_to_bf16(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000f000fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000f000fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000f000fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000f000fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

// Permutation of an 8-element block used for q4 activations: position p holds
// element kPerm[p].
__device__ __forceinline__ uint4 permute8(uint4 v) {
  // elements (bf16) e0..e7 packed as v.x = e0|e1<<16, ...; want e0,e4,e1,e5,e2,e6,e3,e7
  uint4 r;
  r.x = (v.x & 0xffffu) | (v.z << 16);            // e0, e4
  r.y = (v.x >> 16) | (v.z & 0xffff0000u);        // e1, e5
  r.z = (v.y & 0xffffu) | (v.w << 16);            // e2, e6
  r.w = (v.y >> 16) | (v.w & 0xffff0000u);        // e3, e7
  return r;
}

__device__ __forceinline__ float sum8_bf16(uint4 v) {
  return ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
         ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
}

struct GemmArgs {
  const void *act;          // gate/up: x [T][D]; down: h [rows][F] (bf16)
  const int32_t *row_map;   // gate/up only
  int T, N, K;              // token count, routed rows, reduction length
  int n_out;                // output columns of the projection (F for gate/up, D for down)
  int fused;                // gate/up: [gate | up] in one matrix
  int round_ops;            // per-op bf16 SwiGLU
  const void *w0;           // gate (or gate_up) / down weights
  const uint16_t *s0, *b0;
  const void *w1;           // up weights (separate layout)
  const uint16_t *s1, *b1;
  const int32_t *counters;  // [1] = number of tiles
  const PlanItem *tiles;
  void *out;                // gate/up: h bf16 [rows][F]; down: y fp32 [rows][D]
};

// Shared-memory layout of one slab.
template <int RB, int NROWS>
struct Smem {
  uint16_t a[RB * 16][kLdsRow];           // activations (bf16 bits), q4 order inside 8-blocks
  float xg[kGroupsPerSlab][RB * 16];      // group sums of the activations
  float2 sb[kGroupsPerSlab][NROWS];       // (scale, bias - 128*scale) per weight row and group
};

// Token row of tile row m (gate/up), or -1 for padding / out-of-range.
__device__ __forceinline__ int64_t act_row(const GemmArgs &a, const PlanItem &t, int m, bool gateup) {
  if (m >= t.rows) return -1;
  const int p = t.row0 + m;
  if (!gateup) return p;
  const int tok = p < a.N ? a.row_map[p] : (p - a.N) % a.T;
  return unsigned(tok) < unsigned(a.T) ? int64_t(tok) : int64_t(-1);
}

// GATEUP: true -> gate/up projection with SwiGLU epilogue writing h;
//         false -> down projection writing fp32 y rows.
// Q4: affine 4-bit weights; otherwise dense bf16.
// RB: 16-row blocks per tile; NT: 16-row weight tiles per wave (gate/up: NT/2
// gate tiles followed by the NT/2 up tiles of the same columns).
template <bool GATEUP, bool Q4, int RB, int NT>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NW = kThreads / kWave;
  constexpr int NROWS = NW * NT * 16;  // weight rows (incl. up rows) per block
  __shared__ Smem<RB, NROWS> sm;

  if (int(blockIdx.y) >= a.counters[1]) return;
  const PlanItem tile = a.tiles[blockIdx.y];
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int K = a.K, KW = K / 8, G = K / kGroup;
  const int rb_count = (tile.rows + 15) / 16;
  constexpr int NTH = GATEUP ? NT / 2 : NT;
  // First output column of this wave.
  const int col0 = (blockIdx.x * NW + wave) * NTH * 16;

  // Global weight row (expert-major) of weight tile `nt` row r (0..15).
  auto wrow = [&](int nt, int r) -> int64_t {
    const int c = col0 + (nt % NTH) * 16 + r;
    if (!GATEUP) return int64_t(tile.expert) * a.n_out + c;
    const bool up = nt >= NTH;
    if (a.fused) return int64_t(tile.expert) * 2 * a.n_out + (up ? a.n_out : 0) + c;
    return int64_t(tile.expert) * a.n_out + c;
  };
  auto wbase = [&](int nt) -> const void * { return (GATEUP && !a.fused && nt >= NTH) ? a.w1 : a.w0; };
  auto sbase = [&](int nt) -> const uint16_t * { return (GATEUP && !a.fused && nt >= NTH) ? a.s1 : a.s0; };
  auto bbase = [&](int nt) -> const uint16_t * { return (GATEUP && !a.fused && nt >= NTH) ? a.b1 : a.b0; };
  const bool col_ok = col0 < a.n_out;  // whole wave in or out (n_out % 16 == 0)

  f32x4 acc[NT][RB];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[nt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lg = lane >> 4;  // operand row / reduction block of this lane

  for (int k0 = 0; k0 < K; k0 += kKS) {
    const int ks = min(kKS, K - k0);
    __syncthreads();
    // Stage activations: 16-byte pieces of 8 bf16.
    for (int q = tid; q < RB * 16 * (kKS / 8); q += kThreads) {
      const int m = q / (kKS / 8), c8 = q % (kKS / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      const int64_t r = (c8 * 8 < ks) ? act_row(a, tile, m, GATEUP) : -1;
      if (r >= 0) v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + r * K + k0 + c8 * 8);
      if (Q4) v = permute8(v);
      *reinterpret_cast<uint4 *>(&sm.a[m][c8 * 8]) = v;
    }
    if (Q4) {
      // Scales and (bias - 128*scale) of this slab's groups, one weight row per thread.
      for (int r = tid; r < NROWS; r += kThreads) {
        // row r belongs to wave r / (NT*16), weight tile (r / 16) % NT
        const int rw = r / (NT * 16), nt = (r / 16) % NT, rr = r % 16;
        const int c = (blockIdx.x * NW + rw) * NTH * 16 + (nt % NTH) * 16 + rr;
        int64_t wr;
        if (!GATEUP) wr = int64_t(tile.expert) * a.n_out + c;
        else if (a.fused) wr = int64_t(tile.expert) * 2 * a.n_out + (nt >= NTH ? a.n_out : 0) + c;
        else wr = int64_t(tile.expert) * a.n_out + c;
        const int g0 = k0 / kGroup;
        for (int g = 0; g < kGroupsPerSlab; ++g) {
          float2 v = make_float2(0.f, 0.f);
          if (c < a.n_out && g0 + g < G) {
            const float s = bf16_bits_to_f32(sbase(nt)[wr * G + g0 + g]);
            const float b = bf16_bits_to_f32(bbase(nt)[wr * G + g0 + g]);
            v = make_float2(s, __builtin_fmaf(-128.0f, s, b));
          }
          sm.sb[g][r] = v;
        }
      }
    }
    __syncthreads();
    if (Q4) {
      // Group sums of the staged activations (fixed order: deterministic).
      for (int q = tid; q < RB * 16 * kGroupsPerSlab; q += kThreads) {
        const int m = q % (RB * 16), g = q / (RB * 16);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < kGroup / 8; ++j) s += sum8_bf16(*reinterpret_cast<const uint4 *>(&sm.a[m][g * kGroup + j * 8]));
        sm.xg[g][m] = s;
      }
      __syncthreads();
    }
    if (!col_ok) continue;

    for (int g = 0; g < ks / kGroup; ++g) {
      const int kg = k0 + g * kGroup;  // first reduction element of the group
      // Activation operands of the two MFMAs of this group, per row block.
      bf16x8 bx[2][RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < rb_count) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bx[j][rb] = *reinterpret_cast<const bf16x8 *>(&sm.a[rb * 16 + lr][g * kGroup + lg * 16 + j * 8]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t wr = wrow(nt, lr);
        bf16x8 aw[2];
        if constexpr (Q4) {
          const uint2 w2 = *reinterpret_cast<const uint2 *>(static_cast<const uint32_t *>(wbase(nt)) + wr * KW + kg / 8 + lg * 2);
          aw[0] = q4_word_to_bf16(w2.x);
          aw[1] = q4_word_to_bf16(w2.y);
        } else {
          const uint16_t *p = static_cast<const uint16_t *>(wbase(nt)) + wr * K + kg + lg * 16;
          aw[0] = *reinterpret_cast<const bf16x8 *>(p);
          aw[1] = *reinterpret_cast<const bf16x8 *>(p + 8);
        }
        float2 sbv[4];
        if constexpr (Q4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sbv[i] = sm.sb[g][(wave * NT + nt) * 16 + lg * 4 + i];
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (rb < rb_count) {
            if constexpr (Q4) {
              f32x4 d = mfma16(aw[0], bx[0][rb], f32x4{0.f, 0.f, 0.f, 0.f});
              d = mfma16(aw[1], bx[1][rb], d);
              const float xs = sm.xg[g][rb * 16 + lr];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[nt][rb][i] = __builtin_fmaf(sbv[i].y, xs, __builtin_fmaf(sbv[i].x, d[i], acc[nt][rb][i]));
            } else {
              acc[nt][rb] = mfma16(aw[0], bx[0][rb], acc[nt][rb]);
              acc[nt][rb] = mfma16(aw[1], bx[1][rb], acc[nt][rb]);
            }
          }
        }
      }
    }
  }
  if (!col_ok) return;

  // Epilogue: lane holds outputs n = col + lg*4 + i of tile row m = rb*16 + lr.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = rb * 16 + lr;
    if (m >= tile.rows) continue;
    const int64_t row = tile.row0 + m;
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt) {
      const int c = col0 + nt * 16 + lg * 4;
      if constexpr (GATEUP) {
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_bits(swiglu(acc[nt][rb][i], acc[nt + NTH][rb][i], a.round_ops));
        uint2 o = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) = o;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * a.n_out + c) =
            make_float4(acc[nt][rb][0], acc[nt][rb][1], acc[nt][rb][2], acc[nt][rb][3]);
      }
    }
  }
}

template <bool GATEUP, bool Q4, int RB, int NT>
void launch_one(const GemmArgs &ga, int64_t max_tiles, hipStream_t s) {
  constexpr int NTH = GATEUP ? NT / 2 : NT;
  const int cols_per_block = (kThreads / kWave) * NTH * 16;
  const dim3 grid((ga.n_out + cols_per_block - 1) / cols_per_block, unsigned(max_tiles));
  hipLaunchKernelGGL((grouped_gemm_kernel<GATEUP, Q4, RB, NT>), grid, dim3(kThreads), 0, s, ga);
}

}  // namespace

bool use_mfma(const moe_layer_desc *d) {
  // bf16 activations with every reduction length a whole number of 64-element
  // groups; fp32 layers and other shapes take the dequant-GEMV kernels.
  return d->act_dtype == MOE_DT_BF16 && d->d_model % 64 == 0 && d->d_ff % 64 == 0;
}

int plan_tile_rows(const moe_layer_desc *d, int32_t T) {
  // Decode-sized groups (T*k/E <= 8 rows per expert on average, the pages'
  // small-group regime) use 16-row tiles; larger groups 64-row tiles.
  const int64_t N = int64_t(T) * d->top_k;
  return N <= 8LL * d->n_experts ? 16 : 64;
}

void launch_expert_ffn_mfma(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                            const moe_weights *w, const int32_t *counters, const PlanItem *tiles,
                            int64_t max_tiles, void *h, float *y_sorted, void *stream, StageMarker *mk) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool q4 = d->w_format == MOE_WF_AFFINE_Q4;
  const int tr = plan_tile_rows(d, T);
  const moe_proj &pg = d->gate_up_fused ? w->gate_up : w->gate;
  GemmArgs gu{x, row_map, T, T * d->top_k, d->d_model, d->d_ff, d->gate_up_fused, d->swiglu_round_bf16,
              pg.w, static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pg.biases),
              w->up.w, static_cast<const uint16_t *>(w->up.scales), static_cast<const uint16_t *>(w->up.biases),
              counters, tiles, h};
  GemmArgs dn{h, nullptr, T, T * d->top_k, d->d_ff, d->d_model, 0, 0,
              w->down.w, static_cast<const uint16_t *>(w->down.scales), static_cast<const uint16_t *>(w->down.biases),
              nullptr, nullptr, nullptr, counters, tiles, y_sorted};
  if (tr == 16) {
    if (q4) launch_one<true, true, 1, 4>(gu, max_tiles, s);
    else launch_one<true, false, 1, 4>(gu, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    if (q4) launch_one<false, true, 1, 4>(dn, max_tiles, s);
    else launch_one<false, false, 1, 4>(dn, max_tiles, s);
    if (mk) mk->mark("down_mfma");
  } else {
    if (q4) launch_one<true, true, 4, 4>(gu, max_tiles, s);
    else launch_one<true, false, 4, 4>(gu, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    if (q4) launch_one<false, true, 4, 4>(dn, max_tiles, s);
    else launch_one<false, false, 4, 4>(dn, max_tiles, s);
    if (mk) mk->mark("down_mfma");
  }
}

}  // namespace moe
