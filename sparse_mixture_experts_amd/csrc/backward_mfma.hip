// backward_mfma.hip -- the backward pass of 16-bit layers on the matrix cores.
//
// "SwitchGLU: grouped-expert Metal kernels" (ml-explore/mlx-lm #2044),
// section "What": the grouped expert kernels carry a custom VJP.  The pass is
// the chain of contractions of the fp32 vector-unit kernels, over the same
// grouping of sorted rows by expert (the forward's plan tiles):
//   g | u = x Wgu^T     the forward's grouped gate/up GEMM without its GLU
//                       epilogue (x read through row_map, g and u out as fp32)
//   v     = dy Wd       transposed use of the down weights
//   dw, dg | du         per row, from g, u, v and the slot weight (GLU derivative)
//   dx_r  = [dg|du] Wgu transposed use of the gate/up weights
//
// Transposed use.  The stored matrices keep the forward's reduction dimension
// contiguous (codes packed and quantised in groups along a row), so v and
// dx_r reduce over the stored row index.  A workgroup owns one plan tile (up
// to 16*RB rows of one expert), 256 output columns (stored columns, 64 per
// wave) and a range of the reduction.  Each lane loads, straight into
// registers, the words of eight consecutive reduction rows that hold its
// columns, and builds from them operand A of a 16x16x32 MFMA one column at
// a time (see tgemm_body for the lane mapping and the operand formats: fp16
// with power-of-two exponents for affine and fp16 weights, exact bf16
// weights against a bf16 head/tail split of the activations otherwise).
// The activations (dy gathered by token, or the dg|du rows, both fp32) are
// staged in LDS as [rows][64] and read as operand B; fp32 accumulation.
//
// Small row counts split the reduction over several workgroups; each split
// writes its own partial sums and the consumers (the GLU kernel for v, the
// per-token sum for dx) add them in split order, so results do not depend on
// scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

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
constexpr int kWaveCols = 64;                        // output columns per wave
constexpr int kTN = kThreads / kWave * kWaveCols;    // output columns per workgroup (256)
constexpr int kTK = 64;                              // reduction rows per activation slab (two k-blocks of 32)
constexpr int kARow = kTK + 8;                       // bf16 elements per LDS activation row

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- transposed grouped GEMM -------------------------------------------------
struct TArgs {
  const float *act;       // fp32 rows: ASRC 0: dy [T][K] read through the rows' tokens; 1: dg|du [R][K] sorted rows
  const int8_t *act_sh;   // fp16 operands: power-of-two exponent of every activation row (ASRC 0: per token)
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// QB: 4 or 8 (affine codes) or 16 (dense 16-bit weights).  RB: 16-row blocks
// per tile.  ASRC: activation source (see TArgs::act).  HF: scales/biases or
// dense weights are fp16 (else bf16).
//
// Operands.  Affine weights and fp16 dense weights run on the fp16 matrix
// cores: the activations are staged as fp16 scaled by a power of two per row
// (act_sh, undone in the epilogue), and affine codes are expanded to fp16
// s*q + b as in the forward (a code pair placed under the exponent of 1024,
// 1024 subtracted exactly, one packed fma).  A k-block whose scales would
// leave fp16's comfortable range (|s| qmax + |b| of a row at or above 2^15,
// or nonzero below 2^-10) takes one power-of-two exponent for the whole wave
// (the largest of its rows), by which the accumulators are brought to the
// block's scale before its products and back after (exact).  Dense bf16
// weights are exact bf16 operands; their activations are split into a bf16
// head and tail (v = hi + lo with lo = bf16(v - hi)) and multiplied twice.
// Either way both operands carry at least 11 significant bits.
//
// A wave owns 64 output columns and computes them as four MFMA column sets
// of 16.  Lane (m = lane % 16, lg = lane / 16) loads, for each k-block of 32
// reduction rows, the 32-bit word (dword for dense weights) of rows
// 8*lg .. 8*lg+7 that holds its columns, and column set s takes from each of
// those words the value of one column:
//   4-bit: word m % 8 of the wave, nibble 4*(m / 8) + s   (column 8*(m%8) + 4*(m/8) + s)
//   8-bit: word m, byte s                                  (column 4*m + s)
//   dense: dword m + 16*(s/2), half s % 2                  (column 2*(m + 16*(s/2)) + s%2)
// so every lane's operand A of set s is the eight values of one column for
// its eight rows, with no transpose through LDS: for each row pair one byte
// permute brings the pair's bytes side by side, and the codes of both rows
// are expanded together.  (For 4-bit codes lanes m and m + 8 load the same
// word and use its two halves.)  The activations of the tile are staged in
// LDS per slab of 64 reduction rows and read as operand B.
template <int QB, int RB, int ASRC, bool HF>
__device__ __forceinline__ void tgemm_body(const TArgs &a) {
  constexpr bool AFF = QB != 16;
  constexpr bool F16 = AFF || HF;     // fp16 matrix cores (else bf16 weights, split activations)
  constexpr int NPART = F16 ? 1 : 2;  // activation parts in LDS (bf16 head and tail)
  constexpr int VPW = 32 / QB;   // values per 32-bit word (8, 4, 2)
  constexpr int NWL = AFF ? 1 : 2;  // distinct words per row and lane
  constexpr float kQMax = QB == 8 ? 255.0f : 15.0f;
  constexpr int PPR = kTK / 8;    // 8-element activation pieces per row and slab
  constexpr int RPP = kThreads / PPR;
  constexpr int APASS = (RB * 16 + RPP - 1) / RPP;
  __shared__ uint16_t as[2][NPART][RB * 16 * kARow];
  __shared__ int8_t rsh[RB * 16];  // fp16 operands: exponents of the tile's activation rows

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
  PlanItem tile = a.tiles[tile_id];
  // uniform across the workgroup: kept in scalar registers
  tile.expert = __builtin_amdgcn_readfirstlane(tile.expert);
  tile.row0 = __builtin_amdgcn_readfirstlane(tile.row0);
  tile.rows = __builtin_amdgcn_readfirstlane(tile.rows);
  const int ks = a.K / a.ksplit;  // whole slabs (the host picks the split)
  const int k_begin = z * ks, nsl = ks / kTK, nkb = ks / 32;

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int wc0 = cb * kTN + wave * kWaveCols;  // first column of this wave

  // this lane's word column(s) and byte selectors per column set
  const int wpr_row = a.n_cols / VPW;  // words per stored row
  int wcol[NWL];
  if constexpr (QB == 4) wcol[0] = wc0 / 8 + (lr & 7);
  else if constexpr (QB == 8) wcol[0] = wc0 / 4 + lr;
  else {
    wcol[0] = wc0 / 2 + lr;
    wcol[1] = wc0 / 2 + lr + 16;
  }
#pragma unroll
  for (int v = 0; v < NWL; ++v) wcol[v] = min(wcol[v], wpr_row - 1);  // columns past n_cols are never stored
  // Byte permutes that put byte b of a row pair's words (w0 of row 2p, w1 of
  // row 2p + 1) at bytes 0 and 2 of one word: sel(b) = b | (4 + b) << 16,
  // bytes 1 and 3 zero (selector 0x0c).  4-bit: this lane's half word is
  // bytes 2*(m/8) and 2*(m/8) + 1 (column sets 0, 1 and 2, 3); 8-bit: byte s
  // for set s.
  auto byte_sel = [](int b) { return 0x0c000c00u | (uint32_t(4 + b) << 16) | uint32_t(b); };
  const int byte0 = QB == 4 ? 2 * (lr >> 3) : 0;
  const int ngrp = AFF ? a.n_cols / a.group : 1;
  const int grp = AFF ? wcol[0] * VPW / a.group : 0;
  // Addresses: a base common to the workgroup (the expert's matrix, or its
  // scale rows) plus 32-bit per-lane offsets, so that the loads take the
  // scalar-base form.
  const uint32_t *wbase[2];
  const uint32_t *sbase[2], *bbase[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    wbase[mt] = static_cast<const uint32_t *>(a.w[mt]) + int64_t(tile.expert) * a.nre[mt] * wpr_row;
    if constexpr (AFF) {
      sbase[mt] = reinterpret_cast<const uint32_t *>(a.sc[mt] + int64_t(tile.expert) * ngrp * a.nre[mt]);
      bbase[mt] = reinterpret_cast<const uint32_t *>(a.bi[mt] + int64_t(tile.expert) * ngrp * a.nre[mt]);
    }
  }
  uint32_t woff[NWL];  // byte offset of this lane's word in row 8*lg
#pragma unroll
  for (int v = 0; v < NWL; ++v) woff[v] = uint32_t(8 * lg * wpr_row + wcol[v]) * 4u;
  // byte offset of the scale pair (rows 8*lg, 8*lg + 1) of this lane's group, per matrix
  uint32_t soff[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) soff[mt] = uint32_t(grp * a.nre[mt] + 8 * lg) * 2u;
  auto ld = [](const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const uint32_t *>(static_cast<const char *>(base) + byte_off);
  };

  // One k-block's weights in registers: eight rows' words and four
  // (row, row + 1) scale and bias pairs.
  struct WBlock {
    uint32_t w[8][NWL];
    uint32_t s[4], b[4];
  };
  auto load_block = [&](int kb, WBlock &wb) {
    const int k = k_begin + 32 * kb;  // a k-block lies in one matrix (k_second is a multiple of 64)
    const int mt = k >= a.k_second ? 1 : 0;
    const int row = k - (mt ? a.k_second : 0);
    const uint32_t *wp = (mt ? wbase[1] : wbase[0]) + row * wpr_row;  // uniform
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < NWL; ++v) wb.w[i][v] = ld(wp + i * wpr_row, woff[v]);
    if constexpr (AFF) {
      const uint32_t *sp = (mt ? sbase[1] : sbase[0]) + row / 2, *bp = (mt ? bbase[1] : bbase[0]) + row / 2;
      const uint32_t so = mt ? soff[1] : soff[0];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        wb.s[p] = ld(sp + p, so);
        wb.b[p] = ld(bp + p, so);
      }
    }
  };

  // activation staging role: piece pc of rows rr + i*RPP
  const int pc = tid % PPR, rr = tid / PPR;
  int64_t aoff[APASS];
  bool aok[APASS];
  float amul[APASS];  // fp16 operands: 2^-(row exponent)
#pragma unroll
  for (int i = 0; i < APASS; ++i) {
    const int m = rr + i * RPP;
    aok[i] = m < tile.rows && m < RB * 16;
    const int q = tile.row0 + (aok[i] ? m : 0);
    int src = q;
    if constexpr (ASRC == 0) src = q < a.N ? a.row_map[q] : (q - a.N) % a.T;
    aoff[i] = int64_t(src) * a.K + pc * 8;
    amul[i] = 1.0f;
    if constexpr (F16) {
      const int sh = a.act_sh[src];
      amul[i] = pow2(-sh);
      if (pc == 0 && m < RB * 16) rsh[m] = int8_t(aok[i] ? sh : 0);  // visible after the first barrier
    }
  }
  struct AStage {
    float4 f[APASS][2];
  };
  auto load_a = [&](int slab, AStage &st) {
    const int k = k_begin + slab * kTK;
#pragma unroll
    for (int i = 0; i < APASS; ++i) {
      const float4 *p = reinterpret_cast<const float4 *>(a.act + aoff[i] + k);
      st.f[i][0] = p[0];
      st.f[i][1] = p[1];
    }
  };
  auto write_a = [&](const AStage &st, uint16_t (*dst)[RB * 16 * kARow]) {
#pragma unroll
    for (int i = 0; i < APASS; ++i) {
      const int m = rr + i * RPP;
      if (m < RB * 16) {
        const float v[8] = {st.f[i][0].x, st.f[i][0].y, st.f[i][0].z, st.f[i][0].w,
                            st.f[i][1].x, st.f[i][1].y, st.f[i][1].z, st.f[i][1].w};
        uint32_t o[NPART][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (F16) {
            const h2 hv = {(_Float16)(v[2 * j] * amul[i]), (_Float16)(v[2 * j + 1] * amul[i])};
            o[0][j] = __builtin_bit_cast(uint32_t, hv);
          } else {
            const uint32_t hi = pack_bf16(v[2 * j], v[2 * j + 1]);
            o[0][j] = hi;
            o[NPART - 1][j] = pack_bf16(v[2 * j] - bf16_lo(hi), v[2 * j + 1] - bf16_hi(hi));
          }
        }
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          uint4 u = make_uint4(o[part][0], o[part][1], o[part][2], o[part][3]);
          if (!aok[i]) u = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4 *>(dst[part] + m * kARow + pc * 8) = u;
        }
      }
    }
  };

  f32x4 acc[4][RB];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[s2][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t magic = 0x64006400u;  // fp16 exponent of 1024 in both halves
  asm volatile("" : "+v"(magic));

  // One k-block: operand B of every row block from LDS, then per column set
  // operand A and its MFMAs.
  auto compute = [&](const WBlock &wb, const uint16_t (*asl)[RB * 16 * kARow], int kbl, auto nrb_tag) {
    constexpr int NRB = decltype(nrb_tag)::value;
    uint4 xv[NPART][NRB];
#pragma unroll
    for (int part = 0; part < NPART; ++part)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        xv[part][rb] = *reinterpret_cast<const uint4 *>(asl[part] + (rb * 16 + lr) * kARow + 32 * kbl + 8 * lg);
    if constexpr (F16) {
      uint32_t av[4][4];  // [column set][row pair] packed fp16
      int e = 0;          // weight exponent of this k-block (uniform)
      if constexpr (AFF) {
        float sv[8], bv[8], wm = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          sv[2 * p] = HF ? f16_lo(wb.s[p]) : bf16_lo(wb.s[p]);
          sv[2 * p + 1] = HF ? f16_hi(wb.s[p]) : bf16_hi(wb.s[p]);
          bv[2 * p] = HF ? f16_lo(wb.b[p]) : bf16_lo(wb.b[p]);
          bv[2 * p + 1] = HF ? f16_hi(wb.b[p]) : bf16_hi(wb.b[p]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) wm = fmaxf(wm, __builtin_fmaf(kQMax, fabsf(sv[i]), fabsf(bv[i])));
        if (__ballot(f16_shift(wm) != 0)) e = f16_shift(wave_max(wm));
        const float m = pow2(-e);
        h2 s2[4], s2_16[4], b2[4];
        const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          s2[p] = h2{(_Float16)(sv[2 * p] * m), (_Float16)(sv[2 * p + 1] * m)};
          b2[p] = h2{(_Float16)(bv[2 * p] * m), (_Float16)(bv[2 * p + 1] * m)};
          s2_16[p] = s2[p] * sixteenth;
        }
        const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t w0 = wb.w[2 * p][0], w1 = wb.w[2 * p + 1][0];
          if constexpr (QB == 4) {
            // bytes byte0 (sets 0, 1) and byte0 + 1 (sets 2, 3); low nibble
            // gives 1024 + q, high nibble 1024 + 16 q (used with s / 16)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint32_t t = __builtin_amdgcn_perm(w1, w0, byte_sel(byte0 + j));
              const uint32_t clo = (t & 0x000f000fu) | magic, chi = (t & 0x00f000f0u) | magic;
              av[2 * j][p] = __builtin_bit_cast(
                  uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, clo) - k1024, s2[p], b2[p]));
              av[2 * j + 1][p] = __builtin_bit_cast(
                  uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, chi) - k1024, s2_16[p], b2[p]));
            }
          } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const uint32_t c = __builtin_amdgcn_perm(w1, w0, byte_sel(st)) | magic;  // 1024 + q, q <= 255
              av[st][p] = __builtin_bit_cast(
                  uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, c) - k1024, s2[p], b2[p]));
            }
          }
        }
      } else {
        // fp16 dense weights as stored: half st % 2 of dword st / 2 of the row pair
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int st = 0; st < 4; ++st)
            av[st][p] = __builtin_amdgcn_perm(wb.w[2 * p + 1][st >> 1], wb.w[2 * p][st >> 1],
                                              (st & 1) ? 0x07060302u : 0x05040100u);
      }
      if (e != 0) {
        const float m = pow2(-e);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[st][rb] *= m;
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f16x8 wa = __builtin_bit_cast(f16x8, make_uint4(av[st][0], av[st][1], av[st][2], av[st][3]));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[st][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, __builtin_bit_cast(f16x8, xv[0][rb]), acc[st][rb],
                                                               0, 0, 0);
      }
      if (e != 0) {
        const float m = pow2(e);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[st][rb] *= m;
      }
    } else {
      // bf16 dense weights as stored; activation head and tail
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t w0 = wb.w[2 * p][st >> 1], w1 = wb.w[2 * p + 1][st >> 1];
          o[p] = (st & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
        }
        const bf16x8 wa = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          acc[st][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xv[0][rb]),
                                                                acc[st][rb], 0, 0, 0);
          acc[st][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xv[NPART - 1][rb]),
                                                                acc[st][rb], 0, 0, 0);
        }
      }
    }
  };

  // Activations: two LDS buffers, one slab (two k-blocks) ahead in
  // registers.  Weights: a ring of four k-block register sets, loaded two
  // k-blocks ahead of their use (loads past the end repeat the last block).
  // The loop runs for the number of row blocks that hold rows (NRB), so the
  // MFMAs carry no branches.
  auto run = [&](auto nrb_tag) {
    WBlock wb[4];
    AStage ast;
    load_block(0, wb[0]);
    load_block(min(1, nkb - 1), wb[1]);
    load_a(0, ast);
    write_a(ast, as[0]);
    if (nsl > 1) load_a(1, ast);
    __syncthreads();
    for (int i = 0; i < nsl; i += 2) {
      // slab i in buffer 0: k-blocks 2i, 2i+1 in wb[0], wb[1]
      load_block(min(2 * i + 2, nkb - 1), wb[2]);
      compute(wb[0], as[0], 0, nrb_tag);
      load_block(min(2 * i + 3, nkb - 1), wb[3]);
      compute(wb[1], as[0], 1, nrb_tag);
      if (i + 1 < nsl) write_a(ast, as[1]);
      if (i + 2 < nsl) load_a(i + 2, ast);
      __syncthreads();
      if (i + 1 >= nsl) break;
      // slab i+1 in buffer 1: k-blocks 2i+2, 2i+3 in wb[2], wb[3]
      load_block(min(2 * i + 4, nkb - 1), wb[0]);
      compute(wb[2], as[1], 0, nrb_tag);
      load_block(min(2 * i + 5, nkb - 1), wb[1]);
      compute(wb[3], as[1], 1, nrb_tag);
      if (i + 2 < nsl) write_a(ast, as[0]);
      if (i + 3 < nsl) load_a(i + 3, ast);
      __syncthreads();
    }
  };
  if constexpr (RB == 4) {
    const int nrb = (tile.rows + 15) / 16;
    if (nrb >= 4) run(std::integral_constant<int, 4>{});
    else if (nrb == 3) run(std::integral_constant<int, 3>{});
    else if (nrb == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, RB>{});
  }

  // Lane holds, per column set st and row block rb, outputs of tile row
  // rb*16 + lr at the columns of A rows m' = 4*lg + e (e = 0..3); fp16
  // operands: times 2^(the row's activation exponent).
  float *out = a.out + int64_t(z) * a.split_stride;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = rb * 16 + lr;
    if (m >= tile.rows) continue;
    const float rm = F16 ? pow2(rsh[m]) : 1.0f;
    float *orow = out + int64_t(tile.row0 + m) * a.n_cols;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mp = 4 * lg + e;
      if constexpr (QB == 4 || QB == 8) {
        const int c = wc0 + (QB == 4 ? 8 * (mp & 7) + 4 * (mp >> 3) : 4 * mp);
        if (c < a.n_cols)
          *reinterpret_cast<float4 *>(orow + c) =
              make_float4(acc[0][rb][e] * rm, acc[1][rb][e] * rm, acc[2][rb][e] * rm, acc[3][rb][e] * rm);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = wc0 + 2 * (mp + 16 * h);
          if (c < a.n_cols)
            *reinterpret_cast<float2 *>(orow + c) = make_float2(acc[2 * h][rb][e] * rm, acc[2 * h + 1][rb][e] * rm);
        }
      }
    }
  }
}

// 64-row tiles ask for two waves per SIMD (the register budget of the
// accumulators and the weight ring); 16-row tiles allocate on their own.
template <int QB, int RB, int ASRC, bool HF>
__global__ __launch_bounds__(kThreads) void tgemm_kernel(TArgs a) {
  tgemm_body<QB, RB, ASRC, HF>(a);
}
template <int QB, int RB, int ASRC, bool HF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void tgemm_kernel_w2(TArgs a) {
  tgemm_body<QB, RB, ASRC, HF>(a);
}

// Power-of-two exponent of each fp32 row (one wave per row): the fp16
// operand of row r is v * 2^-sh[r] (f16_shift of the row's largest |v|).
__global__ __launch_bounds__(256) void row_exp_f32_kernel(const float *v, int rows, int K, int8_t *sh) {
  const int r = blockIdx.x * (256 / kWave) + int(threadIdx.x) / kWave;
  if (r >= rows) return;  // whole waves
  const float4 *p = reinterpret_cast<const float4 *>(v + int64_t(r) * K);
  float mx = 0.f;
  for (int i = lane_id(); i < K / 4; i += kWave) {
    const float4 q = p[i];
    mx = fmaxf(fmaxf(mx, fmaxf(fabsf(q.x), fabsf(q.y))), fmaxf(fabsf(q.z), fabsf(q.w)));
  }
  mx = wave_max(mx);
  if (lane_id() == 0) sh[r] = int8_t(f16_shift(mx));
}

// ---- GLU backward per sorted row ---------------------------------------------
// dw_r = h . v and dg = c v u a'(g), du = c v a(g), written as fp32 [R][2F]
// (dg then du) with the row's power-of-two exponent for the fp16 operands,
// with v the sum of the split partials.
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
  float *dgu;
  int8_t *dgu_sh;
};
__global__ __launch_bounds__(256) void glu_grad_kernel(GluArgs a) {
  __shared__ float part[256 / kWave], pmax[256 / kWave];
  const int r = blockIdx.x;
  const float c = r < a.N ? a.topk_w[a.order[r]] : 1.0f;
  float dwp = 0.f, mx = 0.f;
  for (int f = threadIdx.x; f < a.F; f += 256) {
    const float g = a.g[int64_t(r) * a.gu_stride + f], u = a.u[int64_t(r) * a.gu_stride + f];
    float v = 0.f;
    for (int z = 0; z < a.vsplit; ++z) v += a.v[z * a.v_split_stride + int64_t(r) * a.F + f];
    float act, dact;
    gate_act_grad(g, a.geglu != 0, act, dact);
    dwp = __builtin_fmaf(act * u, v, dwp);
    const float dh = c * v;
    const float dg = dh * u * dact, du = dh * act;
    a.dgu[int64_t(r) * 2 * a.F + f] = dg;
    a.dgu[int64_t(r) * 2 * a.F + a.F + f] = du;
    mx = fmaxf(mx, fmaxf(fabsf(dg), fabsf(du)));
  }
  dwp = wave_sum(dwp);
  mx = wave_max(mx);
  if (lane_id() == 0) {
    part[threadIdx.x / kWave] = dwp;
    pmax[threadIdx.x / kWave] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.dw[r] = (part[0] + part[1]) + (part[2] + part[3]);
    a.dgu_sh[r] = int8_t(f16_shift(fmaxf(fmaxf(pmax[0], pmax[1]), fmaxf(pmax[2], pmax[3]))));
  }
}

template <int QB, int RB, bool HF>
void launch_t_src(const TArgs &t, int asrc, int64_t max_tiles, hipStream_t s) {
  const dim3 grid(unsigned(((t.n_cols + kTN - 1) / kTN) * t.ksplit), unsigned(max_tiles));
  if constexpr (RB == 1) {
    if (asrc == 0) hipLaunchKernelGGL((tgemm_kernel<QB, RB, 0, HF>), grid, dim3(kThreads), 0, s, t);
    else hipLaunchKernelGGL((tgemm_kernel<QB, RB, 1, HF>), grid, dim3(kThreads), 0, s, t);
  } else {
    if (asrc == 0) hipLaunchKernelGGL((tgemm_kernel_w2<QB, RB, 0, HF>), grid, dim3(kThreads), 0, s, t);
    else hipLaunchKernelGGL((tgemm_kernel_w2<QB, RB, 1, HF>), grid, dim3(kThreads), 0, s, t);
  }
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
  const bool fused = d->gate_up_fused;

  // 1. g | u on the forward's grouped gate/up GEMM ([gate | up] per row)
  launch_gate_up_raw_mfma(d, T, x, row_map, w, counters, tiles, max_tiles, sc.ffn, sc.gu, stream);

  // 2. v = dy Wd (down weights [E+S][D][F]: reduction over d, columns f),
  // dy rows with one power-of-two exponent per token
  hipLaunchKernelGGL(row_exp_f32_kernel, dim3((T + 3) / 4), dim3(256), 0, s, dy, T, D, sc.dy_sh);
  const moe_proj &dn = w->down;
  TArgs tv{dy, sc.dy_sh, row_map, T, N, D, F, D,
           {dn.w, dn.w}, {static_cast<const uint16_t *>(dn.scales), static_cast<const uint16_t *>(dn.scales)},
           {static_cast<const uint16_t *>(dn.biases), static_cast<const uint16_t *>(dn.biases)}, {D, D},
           d->group_size, f16, counters, tiles, sc.v, int64_t(R) * F, sp.v};
  launch_t(tv, qb, tr, 0, max_tiles, s);

  // 3. dw and dg | du per row
  GluArgs ga{sc.gu, sc.gu + F, 2 * F, sc.v, sp.v, int64_t(R) * F, topk_w, order, N, F,
             d->activation == MOE_ACT_GEGLU, sc.dw, sc.dgu, sc.dgu_sh};
  hipLaunchKernelGGL(glu_grad_kernel, dim3(R), dim3(256), 0, s, ga);

  // 4. dx_r = [dg | du] Wgu (gate rows then up rows: reduction over 2F, columns d)
  const moe_proj &pg = fused ? w->gate_up : w->gate, &pu = fused ? w->gate_up : w->up;
  TArgs tx{sc.dgu, sc.dgu_sh, row_map, T, N, 2 * F, D, fused ? 2 * F : F,
           {pg.w, pu.w}, {static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pu.scales)},
           {static_cast<const uint16_t *>(pg.biases), static_cast<const uint16_t *>(pu.biases)},
           {fused ? 2 * F : F, fused ? 2 * F : F}, d->group_size, f16, counters, tiles, sc.dxr, int64_t(R) * D,
           sp.dx};
  launch_t(tx, qb, tr, 1, max_tiles, s);
}

}  // namespace moe
