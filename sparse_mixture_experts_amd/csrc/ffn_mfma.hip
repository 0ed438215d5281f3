// ffn_mfma.hip -- grouped expert GEMMs on the matrix cores (MFMA).
//
// The sorted-row route of DS4Server issue #112 ("Current upstream route",
// "Kernel contract"): workgroups own a tile of one expert's sorted rows; the
// gate/up kernel reads token rows in place through row_map and writes
// silu(gate) * up directly (per-op activation-dtype rounding when asked); the
// down kernel runs on the already sorted, contiguous h rows.  Grouping rows by
// expert means each expert's weights are read and dequantised once per tile
// ("SwitchGLU: grouped-expert Metal kernels", section "What").
//
// gfx950 mapping.  One v_mfma_f32_16x16x32_{f16,bf16} multiplies a 16x32
// weight block (operand A: 16 weight rows n) by a 32x16 activation block
// (operand B: 16 token rows m).  A lane holds row/column l%16 and the 8
// reduction elements 8*(l/16)..+8 of its operand; its 4 results are rows
// n = 4*(l/16)+i of column m = l%16, i.e. 4 consecutive outputs of one token
// row, which makes the stores contiguous.
//
// Weight operands come straight from global memory into registers (every
// weight element is used by exactly one lane), several 64-element groups
// ahead of their use.  Affine 4-bit weights are dequantised in registers to
// fp16 with packed math: for each pair of codes the word is shifted and
// masked into two fp16 values 1024+q (exponent 2^10, the code in the low
// mantissa bits), 1024 is subtracted exactly, and one v_pk_fma_f16 gives
// s*q + b for both.  The pairs come out as (q_j, q_{j+4}) of a word, so the
// activations are staged in LDS with the same order inside every 8-element
// block.  Activations (x or h, bf16) are converted to fp16 when staged.
//
// fp16 has the range of neither bf16 nor the scales, so every staged row gets
// an exponent: activation rows whose largest |value| in the slab reaches 2^15
// are scaled down by a power of two, as are weight rows whose |s|*15 + |b|
// does; a slab in which any row was scaled multiplies the MFMA results by the
// exact power-of-two product before accumulating (the common case, no row
// scaled, accumulates in the MFMA directly).  Dense bf16 weights go to a bf16
// MFMA unchanged.
//
// Activations and scales are staged in LDS in slabs of 128 reduction
// elements, double buffered: the global loads of slab s+1 are in flight in
// registers while slab s is multiplied.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;              // 4 waves
constexpr int kNW = kThreads / kWave;
constexpr int kNT = 4;                     // 16-row weight tiles per wave
constexpr int kNRows = kNW * kNT * 16;     // weight rows per block (256)
constexpr int kKS = 128;                   // reduction elements per slab
constexpr int kGPS = kKS / kGroup;         // groups per slab (2)
constexpr int kLdsRow = kKS + 8;           // padded LDS row (16-bit elements): spreads rows over banks
static_assert(kNRows == kThreads, "one scale row per thread");

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 codes of a word -> 8 fp16 weights s*q + b in the order q0,q4,q1,q5,q2,q6,q3,q7.
__device__ __forceinline__ f16x8 q4_word_to_f16(uint32_t w, h2 s2, h2 b2) {
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  h2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2 q = __builtin_bit_cast(h2, ((w >> (4 * j)) & 0x000f000fu) | 0x64006400u) - k1024;
    r[j] = __builtin_elementwise_fma(q, s2, b2);
  }
  return __builtin_bit_cast(f16x8, r);
}

// 16-bit elements e0..e7 -> e0,e4,e1,e5,e2,e6,e3,e7 (the order of q4_word_to_f16).
__device__ __forceinline__ uint4 permute8(uint4 v) {
  uint4 r;
  r.x = (v.x & 0xffffu) | (v.z << 16);
  r.y = (v.x >> 16) | (v.z & 0xffff0000u);
  r.z = (v.y & 0xffffu) | (v.w << 16);
  r.w = (v.y >> 16) | (v.w & 0xffff0000u);
  return r;
}

// Power-of-two exponent that brings a nonnegative magnitude below 2^15.
__device__ __forceinline__ int f16_shift(float mag) {
  const int ex = int((__float_as_uint(mag) >> 23) & 0xffu) - 127;  // floor(log2(mag)) for normal mag
  return ex >= 15 ? ex - 14 : 0;
}
__device__ __forceinline__ float pow2(int e) { return __uint_as_float(uint32_t(127 + e) << 23); }

// Eight bf16 values scaled by 2^-sh as packed fp16 (two per word).
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 v, int sh) {
  const float m = pow2(-sh);
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 p = {(_Float16)(bf16_lo(u[i]) * m), (_Float16)(bf16_hi(u[i]) * m)};
    o[i] = __builtin_bit_cast(uint32_t, p);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float absmax8_bf16(uint4 v) {
  const float a = fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))), fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  const float b = fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))), fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return fmaxf(a, b);
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

template <int RB>
struct Slab {
  uint16_t a[RB * 16][kLdsRow];   // activations: bf16 (dense) or fp16 in q4 order (q4)
  uint2 sb[kGPS][kNRows];         // q4: (s,s) and (b,b) as packed fp16, per weight row and group
  int8_t ash[RB * 16];            // q4: activation row shifts
  int8_t wsh[kNRows];             // q4: weight row shifts
};

// Per-lane weight data of one group: q4 -> one uint2 per tile; dense -> 2 uint4.
template <bool Q4>
struct WGroup;
template <>
struct WGroup<true> { uint2 w[kNT]; };
template <>
struct WGroup<false> { uint4 w[kNT][2]; };

// GATEUP: gate/up projection with SwiGLU epilogue writing h, else down
// projection writing fp32 y rows.  Q4: affine 4-bit weights (fp16 MFMA),
// else dense bf16 (bf16 MFMA).  RB: 16-row blocks per tile.  Each wave owns
// kNT weight tiles of 16 rows; for gate/up the first kNT/2 are gate rows and
// the last kNT/2 the up rows of the same output columns.
template <bool GATEUP, bool Q4, int RB>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NTH = GATEUP ? kNT / 2 : kNT;  // output-column tiles per wave
  constexpr int TPR = 16 / RB;                 // staging threads per activation row
  constexpr int PPT = RB;                      // 8-element pieces per staging thread
  static_assert(RB * 16 * TPR == kThreads, "staging covers the slab");
  __shared__ Slab<RB> sm[2];

  // XCD-aware order.  Workgroups go to the 8 XCDs round-robin by linear id;
  // the W = tiles * column-blocks work items of this call are cut into 8
  // contiguous ranges, one per XCD, so the column blocks of a tile (which
  // stage the same activation rows) share an L2 and every XCD gets an equal
  // share.  Linear ids past the 8 ranges exit.
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
  const int tile_id = item / nbx, bx = item % nbx;
  const PlanItem tile = a.tiles[tile_id];

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;  // operand row / reduction block of this lane
  const int K = a.K, KW = K / 8, G = K / kGroup;
  const int nslab = (K + kKS - 1) / kKS;
  const int rb_count = (tile.rows + 15) / 16;
  const int col0 = (bx * kNW + wave) * NTH * 16;  // first output column of this wave
  const bool col_ok = col0 < a.n_out;              // whole wave in or out (n_out % 64 == 0)

  auto wrow_of = [&](int col, bool up) -> int64_t {
    if (!GATEUP) return int64_t(tile.expert) * a.n_out + col;
    if (a.fused) return int64_t(tile.expert) * 2 * a.n_out + (up ? a.n_out : 0) + col;
    return int64_t(tile.expert) * a.n_out + col;
  };
  auto wsrc = [&](bool up) -> const void * { return (GATEUP && !a.fused && up) ? a.w1 : a.w0; };
  auto ssrc = [&](bool up) -> const uint16_t * { return (GATEUP && !a.fused && up) ? a.s1 : a.s0; };
  auto bsrc = [&](bool up) -> const uint16_t * { return (GATEUP && !a.fused && up) ? a.b1 : a.b0; };

  // Every global load below is issued unconditionally, from a clamped and
  // always valid address (unused data is discarded with a select): loads that
  // sit on only one side of a branch make the compiler wait for all
  // outstanding loads at the join, which would drain the prefetch pipeline.
  const int col_c = col_ok ? col0 : a.n_out - NTH * 16;  // in-range columns for idle waves

  // This lane's weight row (operand A row lr) of each tile.
  int64_t wr[kNT];
  const void *wp[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const bool up = GATEUP && nt >= NTH;
    wr[nt] = wrow_of(col_c + (nt % NTH) * 16 + lr, up);
    wp[nt] = wsrc(up);
  }
  auto load_group = [&](int g, WGroup<Q4> &dst) {
    g = min(g, G - 1);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      if constexpr (Q4) {
        dst.w[nt] = *reinterpret_cast<const uint2 *>(static_cast<const uint32_t *>(wp[nt]) + wr[nt] * KW + g * 8 + lg * 2);
      } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(wp[nt]) + wr[nt] * K + g * kGroup + lg * 16);
        dst.w[nt][0] = p[0];
        dst.w[nt][1] = p[1];
      }
    }
  };

  // ---- staging: thread -> (row m, pieces j*PPT..+PPT of the slab) ----
  const int sm_row = tid / TPR, sj = tid % TPR;
  int64_t src_row = -1;
  if (sm_row < tile.rows) {
    const int p = tile.row0 + sm_row;
    if (!GATEUP) {
      src_row = p;
    } else {
      const int tok = p < a.N ? a.row_map[p] : (p - a.N) % a.T;
      src_row = unsigned(tok) < unsigned(a.T) ? tok : -1;
    }
  }
  const int64_t src_row_c = src_row >= 0 ? src_row : (GATEUP ? 0 : tile.row0);
  // scale row of this thread (one weight row of the block per thread)
  const int s_w = tid / (kNT * 16), s_nt = (tid / 16) % kNT, s_r = tid % 16;
  const int s_col = (bx * kNW + s_w) * NTH * 16 + (s_nt % NTH) * 16 + s_r;
  const bool s_up = GATEUP && s_nt >= NTH;
  const bool s_ok = s_col < a.n_out;
  const int64_t s_wrow = wrow_of(s_ok ? s_col : a.n_out - 1, s_up);

  uint4 stg[PPT];
  uint16_t sraw[kGPS][2];
  auto stage_load = [&](int s) {
    s = min(s, nslab - 1);
    const int k0 = s * kKS;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int k = k0 + (sj * PPT + p) * 8;
      const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + src_row_c * K +
                                                       min(k, K - 8));
      const bool ok = src_row >= 0 && k < K;
      stg[p] = make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    }
    if constexpr (Q4) {
#pragma unroll
      for (int g = 0; g < kGPS; ++g) {
        const int gg = s * kGPS + g;
        const bool ok = s_ok && gg < G;
        const int64_t at = s_wrow * G + min(gg, G - 1);
        const uint16_t sv = ssrc(s_up)[at], bv = bsrc(s_up)[at];
        sraw[g][0] = ok ? sv : uint16_t(0);
        sraw[g][1] = ok ? bv : uint16_t(0);
      }
    }
  };
  // Writes the staged slab to LDS buffer `buf`; returns nonzero when a row of
  // it needed a power-of-two shift to fit fp16.
  auto stage_write = [&](int buf) -> int {
    Slab<RB> &S = sm[buf];
    int flag = 0;
    if constexpr (Q4) {
      float mx = 0.f;
#pragma unroll
      for (int p = 0; p < PPT; ++p) mx = fmaxf(mx, absmax8_bf16(stg[p]));
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      const int sh = f16_shift(mx);
#pragma unroll
      for (int p = 0; p < PPT; ++p)
        *reinterpret_cast<uint4 *>(&S.a[sm_row][(sj * PPT + p) * 8]) = permute8(bf16x8_to_f16(stg[p], sh));
      if (sj == 0) S.ash[sm_row] = int8_t(sh);
      float sv[kGPS], bv[kGPS], wm = 0.f;
#pragma unroll
      for (int g = 0; g < kGPS; ++g) {
        sv[g] = bf16_bits_to_f32(sraw[g][0]);
        bv[g] = bf16_bits_to_f32(sraw[g][1]);
        wm = fmaxf(wm, __builtin_fmaf(15.0f, fabsf(sv[g]), fabsf(bv[g])));
      }
      const int wsh = f16_shift(wm);
      const float m = pow2(-wsh);
#pragma unroll
      for (int g = 0; g < kGPS; ++g) {
        const _Float16 sh16 = (_Float16)(sv[g] * m), bh16 = (_Float16)(bv[g] * m);
        const h2 s2 = {sh16, sh16}, b2 = {bh16, bh16};
        S.sb[g][tid] = make_uint2(__builtin_bit_cast(uint32_t, s2), __builtin_bit_cast(uint32_t, b2));
      }
      S.wsh[tid] = int8_t(wsh);
      flag = sh | wsh;
    } else {
#pragma unroll
      for (int p = 0; p < PPT; ++p) *reinterpret_cast<uint4 *>(&S.a[sm_row][(sj * PPT + p) * 8]) = stg[p];
    }
    return flag;
  };

  f32x4 acc[kNT][RB];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[nt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A slab in which some row was shifted: the accumulators are brought to the
  // slab's scale (times 2^-(activation shift + weight shift) of each output)
  // before its groups accumulate, and back (times 2^+shift) after, both exact.
  auto rescale = [&](const Slab<RB> &S, int sign) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int ash = S.ash[rb * 16 + lr];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[nt][rb][i] *= pow2(sign * (ash + S.wsh[(wave * kNT + nt) * 16 + lg * 4 + i]));
    }
  };

  auto compute_group = [&](const Slab<RB> &S, int gi, const WGroup<Q4> &wg) {
    if constexpr (Q4) {
      f16x8 bx[2][RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb < rb_count)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bx[j][rb] = *reinterpret_cast<const f16x8 *>(&S.a[rb * 16 + lr][gi * kGroup + lg * 16 + j * 8]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const uint2 sbv = S.sb[gi][(wave * kNT + nt) * 16 + lr];
        const h2 s2 = __builtin_bit_cast(h2, sbv.x), b2 = __builtin_bit_cast(h2, sbv.y);
        const f16x8 aw0 = q4_word_to_f16(wg.w[nt].x, s2, b2);
        const f16x8 aw1 = q4_word_to_f16(wg.w[nt].y, s2, b2);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (rb < rb_count) {
            acc[nt][rb] = mfma_f16(aw0, bx[0][rb], acc[nt][rb]);
            acc[nt][rb] = mfma_f16(aw1, bx[1][rb], acc[nt][rb]);
          }
        }
      }
    } else {
      bf16x8 bx[2][RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb < rb_count)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bx[j][rb] = *reinterpret_cast<const bf16x8 *>(&S.a[rb * 16 + lr][gi * kGroup + lg * 16 + j * 8]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const bf16x8 aw0 = __builtin_bit_cast(bf16x8, wg.w[nt][0]);
        const bf16x8 aw1 = __builtin_bit_cast(bf16x8, wg.w[nt][1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (rb < rb_count) {
            acc[nt][rb] = mfma_bf16(aw0, bx[0][rb], acc[nt][rb]);
            acc[nt][rb] = mfma_bf16(aw1, bx[1][rb], acc[nt][rb]);
          }
        }
      }
    }
  };

  // ---- pipelined main loop ----
  // Weights run PD groups ahead in a ring of register buffers (4-bit groups
  // are small, so more of them are kept in flight); the activation slab s+1
  // is loaded during the first group of slab s and written to the other LDS
  // buffer after its last group.  Steps past the last group (when G is not a
  // multiple of PD) only keep the barrier pattern; their loads are clamped
  // repeats and their compute is skipped.
  constexpr int PD = 2;
  static_assert(PD % kGPS == 0, "ring covers whole slabs");
  WGroup<Q4> wb[PD];
  stage_load(0);
  const int f0 = stage_write(0);
#pragma unroll
  for (int u = 0; u < PD; ++u) load_group(u, wb[u]);
  int slow = __syncthreads_or(f0);
  for (int g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int g = g0 + u;
      const int s = g / kGPS, gi = g % kGPS, buf = s & 1;
      if (gi == 0) stage_load(s + 1);
      if (Q4 && slow && gi == 0 && col_ok) rescale(sm[buf], -1);
      if (col_ok && g < G) compute_group(sm[buf], gi, wb[u]);
      load_group(g + PD, wb[u]);
      if (gi == kGPS - 1) {
        if (Q4 && slow && col_ok) rescale(sm[buf], +1);
        slow = __syncthreads_or(stage_write(buf ^ 1));
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
        const uint2 o = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) = o;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * a.n_out + c) =
            make_float4(acc[nt][rb][0], acc[nt][rb][1], acc[nt][rb][2], acc[nt][rb][3]);
      }
    }
  }
}

template <bool GATEUP, bool Q4, int RB>
void launch_one(const GemmArgs &ga, int64_t max_tiles, hipStream_t s) {
  constexpr int NTH = GATEUP ? kNT / 2 : kNT;
  const int cols_per_block = kNW * NTH * 16;
  const dim3 grid((ga.n_out + cols_per_block - 1) / cols_per_block, unsigned(max_tiles));
  hipLaunchKernelGGL((grouped_gemm_kernel<GATEUP, Q4, RB>), grid, dim3(kThreads), 0, s, ga);
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
    if (q4) launch_one<true, true, 1>(gu, max_tiles, s);
    else launch_one<true, false, 1>(gu, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    if (q4) launch_one<false, true, 1>(dn, max_tiles, s);
    else launch_one<false, false, 1>(dn, max_tiles, s);
    if (mk) mk->mark("down_mfma");
  } else {
    if (q4) launch_one<true, true, 4>(gu, max_tiles, s);
    else launch_one<true, false, 4>(gu, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    if (q4) launch_one<false, true, 4>(dn, max_tiles, s);
    else launch_one<false, false, 4>(dn, max_tiles, s);
    if (mk) mk->mark("down_mfma");
  }
}

}  // namespace moe
