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
// weight element is used by exactly one lane), a group ahead of their use.
// Affine 4- and 8-bit weights are dequantised in registers to fp16 with
// packed math: each pair of codes is moved into two fp16 values 1024+q
// (exponent 2^10, the code in the low mantissa bits; 4-bit codes by shift and
// mask, 8-bit codes by byte permutes), 1024 is subtracted exactly, and one
// v_pk_fma_f16 gives s*q + b for both.  The pairs come out as (q_j, q_{j+4})
// of each 8-code block, so the activations are stored with the same order
// inside every 8-element block.
//
// Affine layers keep their activations in fp16 end to end: a small kernel
// converts x once per token (not once per expert tile) and the gate/up
// epilogue writes h as fp16, both already in that permuted order, so the
// GEMMs' LDS staging is a plain copy.  fp16 has the range of neither bf16
// nor the scales, so values carry power-of-two exponents, used only where
// needed: one per token row of x (undone in the gate/up epilogue), one per
// (row, 128-column block) of h, and one per (weight row, slab) for scales
// whose |s|*qmax + |b| (qmax = 15 or 255) is at least 2^15 or below 2^-10.  The main loop runs
// without any rescaling; if a slab of the tile carries an h or weight
// exponent, the tile starts over in a loop that brings the accumulators to
// each such slab's scale and back (exact power-of-two multiplies).  Dense
// bf16 weights go to a bf16 MFMA unchanged.
//
// Activations and scales are staged in LDS in slabs of 128 reduction
// elements, double buffered: the global loads of slab s+1 are in flight in
// registers while slab s is multiplied.
#include <stdexcept>
#include <type_traits>

#include "device_common.h"
#include "dequant_f16.h"
#include "f16_stage.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;              // 4 waves
constexpr int kNW = kThreads / kWave;
constexpr int kNT = 4;                     // 16-row weight tiles per wave
constexpr int kNRows = kNW * kNT * 16;     // weight rows per block (256)
constexpr int kKS = 128;                   // reduction elements per slab
constexpr int kSteps = kKS / 32;           // MFMA reduction steps per slab (4)
constexpr int kPieces = kKS / 8;           // 16-byte activation pieces per row and slab (16)
constexpr int kLdsRow = kKS + 8;           // padded LDS row (16-bit elements): spreads rows over banks
static_assert(kNRows == kThreads, "one scale row per thread");
static_assert(kKS == 32 * 4, "a lane's 4 reduction blocks of 32 span the slab");

// x [T][D] (bf16, or fp16 when x_f16) -> fp16 staging copy (row_to_f16) and
// its group means when xo.xg is set, one wave per token.
__global__ __launch_bounds__(256) void act_f16_kernel(const uint16_t *x, int T, int D, uint16_t *x16,
                                                      int8_t *xsh, int x_f16, XgOut xo) {
  const int t = blockIdx.x * (256 / kWave) + int(threadIdx.x) / kWave;
  if (t >= T) return;  // whole waves
  row_to_f16(x + int64_t(t) * D, D, x16 + int64_t(t) * D, xsh + t, x_f16 != 0, xo, t);
}

struct GemmArgs {
  const void *act;          // gate/up: x [T][K] (bf16; fp16 copy for affine); down: h [rows][K]
  const int8_t *act_sh;     // affine: gate/up token exponents [T]; down h exponents [rows][nblk]
  int8_t *out_sh;           // affine gate/up: h exponents [rows][nblk]; down: y exponents [rows][n_out/64] (or null)
  int nblk;                 // h exponent blocks per row
  const int32_t *row_map;   // gate/up only
  int T, N, K;              // token count, routed rows, reduction length
  int n_out;                // output columns of the projection (F for gate/up, D for down)
  int fused;                // gate/up: [gate | up] in one matrix
  int round_ops;            // per-op GLU rounding mode (kRoundNone / BF16 / F16)
  int geglu;                // gate/up: tanh-GELU gate (else SiLU)
  int half_f16;             // affine scales/biases are fp16 (else bf16)
  const void *w0;           // gate (or gate_up) / down weights
  const uint16_t *s0, *b0;
  const void *w1;           // up weights (separate layout)
  const uint16_t *s1, *b1;
  const int32_t *counters;  // [1] = number of tiles
  const PlanItem *tiles;
  void *out;                // gate/up: h [rows][F] (bf16, or fp16 for affine); down: y [rows][D], fp16 with
                            // exponents when out_sh is set, else fp32
  int bx_major;             // work order: column block major (experts with several tiles), else tile major
  int kz;                   // down: reduction parts (fp32 partial rows at out + z * part_stride), else 1
  int64_t part_stride;
  // affine: tile-packed copies of w0 / w1 (moe_pack_weights), or null; set
  // together (w1's when gate and up are separate)
  const uint32_t *wp0 = nullptr, *wp1 = nullptr;
  // gate/up on packed copies: their fp16 scales, group terms and flags, and
  // the group means of the staged token rows ([T][gp] fp16); xg null: the
  // fast path is off
  const uint16_t *sp0 = nullptr, *sp1 = nullptr, *bp0 = nullptr, *bp1 = nullptr;
  const int32_t *fl0 = nullptr, *fl1 = nullptr;
  const uint16_t *xg = nullptr;
  int gp = 0;
};

// Column blocks per group of the work order (item_tile_block): whole rows of
// blocks (tile-major) when every expert has about one tile; groups of
// kColGroup blocks when the plan finds experts with several tiles (the skewed
// 256-token layer: down read 1.84x its bytes tile-major, 1.18x in groups);
// single blocks (column-block-major: every tile for one block of columns,
// then the next) when the host's layer shape gives every expert two or more
// tiles (the dense 512-token layer: gate/up read 1.22x its bytes this way,
// 1.48x in groups of 8).
__device__ __forceinline__ int col_group(const GemmArgs &a, int nbx) {
  return a.bx_major ? 1 : a.counters[2] ? min(nbx, kColGroup) : nbx;
}

// GPS: groups per slab (128 / group size; 1 for dense weights).
template <int RB, int GPS>
struct Slab {
  uint16_t a[RB * 16][kLdsRow];   // activations: bf16 (dense) or fp16 in permuted order (affine)
  uint2 sb[GPS][kNRows];          // affine: (s,s) and (b,b) as packed fp16, per weight row and group
  int8_t ash[RB * 16];            // affine down: h exponents of the slab's rows
  int8_t wsh[kNRows];             // affine: weight row exponents
};

// Weight formats of the grouped GEMM: QB = 4 or 8 (affine codes, fp16
// MFMA), kDenseBF16 or kDenseF16 (16-bit weights fed to the MFMA as stored).
constexpr int kDenseBF16 = 0, kDenseF16 = 16;
constexpr bool is_affine(int qb) { return qb == 4 || qb == 8; }

// Projections of the grouped GEMM: down (sorted h rows -> y rows), gate/up
// with the GLU epilogue (x rows through row_map -> h), and gate/up with the
// gate and up values written as they are (fp32 rows [gate | up], for the
// backward pass).
constexpr int kDown = 0, kGateUp = 1, kGateUpRaw = 2;

// Per-lane weight data of one slab (32 reduction elements per tile): 4-bit
// -> one uint4 (4 words) per tile; 8-bit -> two; 16-bit dense -> four.
template <int QB>
struct WSlab {
  uint4 w[kNT][is_affine(QB) ? QB / 4 : kSteps];
  uint32_t s[kNT];  // fast path: the lane's fp16 scale of each tile
};

// GATEUP: gate/up projection with the GLU epilogue writing h, else down
// projection writing y rows.  QB: affine code width 4 or 8 (fp16 MFMA), or
// kDenseBF16 / kDenseF16 for 16-bit dense weights (bf16 / fp16 MFMA; h is
// written in that dtype).  RB: 16-row blocks per tile.  GPS:
// affine groups per 128-element slab (4, 2, 1 for groups of 32, 64, 128).  Each wave owns
// kNT weight tiles of 16 rows; for gate/up the first kNT/2 are gate rows and
// the last kNT/2 the up rows of the same output columns.
//
// Reduction order inside a slab of 128: lane (lr, lg) of an operand holds
// the 32 slab elements 32*lg .. 32*lg+31 (4-bit: words 4*lg .. 4*lg+3 of the
// row's slab, one contiguous 16-byte load; 8-bit: words 8*lg .. 8*lg+7), and
// MFMA step j multiplies the 8 elements 32*lg + 8*j .. +7 of both operands.
// Both operands use the same order, so every step sums over a fixed quarter
// of the slab and the four steps cover it.  A lane's 32 elements lie in one
// group: group 32*lg / (128 / GPS) of the slab.
template <int MODE, int QB, int RB, int GPS>
__device__ __forceinline__ void grouped_gemm_body(const GemmArgs &a) {
  constexpr bool GATEUP = MODE != kDown;  // gate/up rows (two weight matrices per column)
  constexpr bool RAW = MODE == kGateUpRaw;  // g and u out as fp32, no GLU
  constexpr bool AFF = is_affine(QB);              // affine codes (fp16 path)
  constexpr int kLPG = 4 / GPS;                   // lanes lg per group
  constexpr float kQMax = QB == 8 ? 255.0f : 15.0f;
  constexpr int NTH = GATEUP ? kNT / 2 : kNT;   // output-column tiles per wave
  constexpr int kRowsPerPass = kThreads / kPieces;  // activation rows staged per pass (16)
  constexpr int PPT = RB * 16 / kRowsPerPass;     // staging passes (pieces per thread)
  static_assert(PPT * kRowsPerPass == RB * 16, "staging covers the slab");
  static_assert(!GATEUP || kNW * NTH * 16 == kHBlock, "a gate/up block writes one h exponent block");
  static_assert(kKS == kHBlock, "a down slab reads one h exponent block");
  __shared__ Slab<RB, GPS> sm[2];
  __shared__ float rmax[GATEUP && AFF ? kNW : 1][RB * 16];  // gate/up affine epilogue: row maxima per wave
  __shared__ int8_t rsh[RB * 16];                         // gate/up affine: token exponents of the rows

  // XCD-aware order.  Workgroups go to the 8 XCDs round-robin by linear id;
  // the W = tiles * column-blocks work items of this call are cut into 8
  // contiguous ranges, one per XCD, so the column blocks of a tile (which
  // stage the same activation rows) share an L2 and every XCD gets an equal
  // share.  Linear ids past the 8 ranges exit.
  const int nbx = gridDim.x;
  const int total = nbx * gridDim.y * gridDim.z;
  const int n_tiles = a.counters[1];
  const int work = n_tiles * nbx * a.kz;
  const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * nbx + blockIdx.x;
  const int per = (work + 7) / 8;
  int item = lin;
  if (8 * per <= total) {
    const int slot = lin / 8;
    if (slot >= per) return;
    item = (lin % 8) * per + slot;
  }
  if (item >= work) return;
  // reduction part (outermost), then the tile and column block.  Tile-major
  // order puts the column blocks of a tile next to each other (they stage
  // the same activation rows); with experts of several tiles, groups of 8
  // column blocks also put the tiles of one expert together (they read the
  // same weights).
  const int z = item / (n_tiles * nbx);
  item -= z * n_tiles * nbx;
  int tile_id, bx;
  item_tile_block(item, n_tiles, nbx, col_group(a, nbx), tile_id, bx);
  const PlanItem tile = a.tiles[tile_id];

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;  // operand row / reduction quarter of this lane
  const int K = a.K, KW = AFF ? K * QB / 32 : 0, G = K / (kKS / GPS);
  // this part's slabs: sbeg .. sbeg + nslab - 1 (the host keeps every part non-empty)
  const int nslab_all = (K + kKS - 1) / kKS, ns = (nslab_all + a.kz - 1) / a.kz;
  const int sbeg = z * ns, nslab = min(ns, nslab_all - sbeg);
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
  // With a tile-packed copy, a lane's row of a slab sits at (tile of 16
  // rows, slab, row in tile): the 16 rows of a slab are one contiguous block.
  constexpr int SW = kKS * QB / 32;  // affine: words of one row's slab
  const bool packed = AFF && a.wp0 != nullptr;
  const void *wp[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const bool up = GATEUP && nt >= NTH;
    const int64_t wr = wrow_of(col_c + (nt % NTH) * 16 + lr, up);
    if (packed) {
      const uint32_t *pb = (GATEUP && !a.fused && up) ? a.wp1 : a.wp0;
      wp[nt] = pb + (wr >> 4) * (int64_t((K + kKS - 1) / kKS) * 16 * SW) + (wr & 15) * SW;
    } else {
      wp[nt] = AFF ? static_cast<const void *>(static_cast<const uint32_t *>(wsrc(up)) + wr * KW)
                  : static_cast<const void *>(static_cast<const uint16_t *>(wsrc(up)) + wr * K);
    }
  }
  // The fast path: gate/up on packed copies whose matrices all
  // carry the flag (and with the token group sums at hand).  Each wave's
  // tiles are addressed through their wave-uniform tile index, so only the
  // lane's offset inside a (tile, slab) block lives in a vector register.
  bool fast = false;
  if constexpr (AFF && GATEUP) {
    if (packed && a.xg)
      fast = __builtin_amdgcn_readfirstlane(a.fl0[tile.expert] != 0 && (a.fused || a.fl1[tile.expert] != 0));
  }
  int ptile[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
    ptile[nt] = __builtin_amdgcn_readfirstlane(int(wrow_of(col_c + (nt % NTH) * 16, GATEUP && nt >= NTH) >> 4));
  constexpr int kGPS = GPS;
  const uint32_t lane_w = uint32_t(lr * SW + lg * (AFF ? QB : 0));  // words
  const uint32_t lane_s = uint32_t(lr * kGPS + lg / kLPG);          // fp16 scales
  auto load_slab_fast = [&](int s, WSlab<QB> &dst) {
    s = sbeg + min(s, nslab - 1);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const bool second = GATEUP && !a.fused && nt >= NTH;
      const int64_t blk = int64_t(ptile[nt]) * nslab_all + s;
      const uint32_t *cb = (second ? a.wp1 : a.wp0) + blk * (16 * SW);
#pragma unroll
      for (int v = 0; v < (AFF ? QB / 4 : 1); ++v) dst.w[nt][v] = *reinterpret_cast<const uint4 *>(cb + lane_w + 4 * v);
      dst.s[nt] = (second ? a.sp1 : a.sp0)[blk * (16 * kGPS) + lane_s];
    }
  };

  // Slab s of this lane's rows.  The last slab may hold only 64 elements
  // (K = 64 mod 128): its second half is read from a clamped address and
  // multiplied by zero scales (affine) or zeroed activations (dense).
  auto load_slab = [&](int s, WSlab<QB> &dst) {
    s = sbeg + min(s, nslab - 1);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      if constexpr (AFF) {
        constexpr int WPL = QB;  // words per lane and slab (32 elements)
        const int w = packed ? s * 16 * SW + lg * WPL : min(s * SW + lg * WPL, KW - WPL);
#pragma unroll
        for (int v = 0; v < QB / 4; ++v)
          dst.w[nt][v] = *reinterpret_cast<const uint4 *>(static_cast<const uint32_t *>(wp[nt]) + w + 4 * v);
      } else {
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
          const int k = min(s * kKS + lg * 32 + j * 8, K - 8);
          dst.w[nt][j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(wp[nt]) + k);
        }
      }
    }
  };

  // ---- staging: pass p of thread tid -> row p*16 + tid/16, piece tid%16 ----
  // (16 consecutive lanes read one row's 256 contiguous bytes of the slab.)
  const int piece = tid % kPieces;
  int src_row[PPT];       // source row, -1 past the tile (or for an invalid token)
  int64_t src_off[PPT];   // element offset of a valid source row
#pragma unroll
  for (int p = 0; p < PPT; ++p) {
    const int m = p * kRowsPerPass + tid / kPieces;
    int r = -1;
    if (m < tile.rows) {
      const int q = tile.row0 + m;
      if (!GATEUP) {
        r = q;
      } else {
        const int tok = q < a.N ? a.row_map[q] : (q - a.N) % a.T;
        r = unsigned(tok) < unsigned(a.T) ? tok : -1;
      }
    }
    src_row[p] = r;
    // Rows past the tile (and invalid tokens) read a valid row; their results
    // are never stored.
    src_off[p] = int64_t(r >= 0 ? r : (GATEUP ? 0 : tile.row0)) * K;
    if constexpr (GATEUP && AFF) {
      if (piece == 0) rsh[m] = a.act_sh[src_off[p] / K];  // visible after the first barrier
    }
  }
  // scale row of this thread (one weight row of the block per thread)
  const int s_w = tid / (kNT * 16), s_nt = (tid / 16) % kNT, s_r = tid % 16;
  const int s_col = (bx * kNW + s_w) * NTH * 16 + (s_nt % NTH) * 16 + s_r;
  const bool s_up = GATEUP && s_nt >= NTH;
  const bool s_ok = s_col < a.n_out;
  // Scales and biases are group-major, [expert][group][row of the expert's
  // matrix], so a wave's loads of one group cover consecutive rows.
  const int s_nre = (GATEUP && a.fused) ? 2 * a.n_out : a.n_out;  // rows of one expert's matrix
  const int s_rin = (GATEUP && a.fused && s_up ? a.n_out : 0) + (s_ok ? s_col : a.n_out - 1);
  const int64_t s_base = int64_t(tile.expert) * G * s_nre + s_rin;

  uint4 stg[PPT];
  uint16_t sraw[GPS][2];
  int stg_sh[PPT];  // affine down: h exponents of the staged rows' slab
  auto stage_load = [&](int s, auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    s = sbeg + min(s, nslab - 1);
    const int k = s * kKS + piece * 8;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + src_off[p] +
                                                       min(k, K - 8));
      if constexpr (AFF) {
        stg[p] = v;  // pieces past K meet zero scales
      } else {
        const bool ok = src_row[p] >= 0 && k < K;
        stg[p] = make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
      }
      if constexpr (AFF && !GATEUP) stg_sh[p] = a.act_sh[(src_off[p] / K) * a.nblk + s];
    }
    if constexpr (AFF && !FAST) {
#pragma unroll
      for (int g = 0; g < GPS; ++g) {
        const int gg = s * GPS + g;
        const bool ok = s_ok && gg < G;
        const int64_t at = s_base + int64_t(min(gg, G - 1)) * s_nre;
        const uint16_t sv = ssrc(s_up)[at], bv = bsrc(s_up)[at];
        sraw[g][0] = ok ? sv : uint16_t(0);
        sraw[g][1] = ok ? bv : uint16_t(0);
      }
    }
  };
  // Writes the staged slab to LDS buffer `buf`; returns nonzero when the slab
  // carries an exponent (h rows of the down projection, or weight rows).
  auto stage_write = [&](int buf, auto fast_tag) -> int {
    constexpr bool FAST = decltype(fast_tag)::value;
    Slab<RB, GPS> &S = sm[buf];
    int flag = 0;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int m = p * kRowsPerPass + tid / kPieces;
      *reinterpret_cast<uint4 *>(&S.a[m][piece * 8]) = stg[p];
      if constexpr (AFF && !GATEUP) {
        const int sh = src_row[p] >= 0 ? stg_sh[p] : 0;
        if (piece == 0) S.ash[m] = int8_t(sh);
        flag |= sh;
      }
    }
    if constexpr (AFF && !FAST) {
      float sv[GPS], bv[GPS], wm = 0.f;
#pragma unroll
      for (int g = 0; g < GPS; ++g) {
        sv[g] = a.half_f16 ? f16_bits_to_f32(sraw[g][0]) : bf16_bits_to_f32(sraw[g][0]);
        bv[g] = a.half_f16 ? f16_bits_to_f32(sraw[g][1]) : bf16_bits_to_f32(sraw[g][1]);
        wm = fmaxf(wm, __builtin_fmaf(kQMax, fabsf(sv[g]), fabsf(bv[g])));
      }
      const int wsh = f16_shift(wm);
      const float m = pow2(-wsh);
#pragma unroll
      for (int g = 0; g < GPS; ++g) {
        const _Float16 sh16 = (_Float16)(sv[g] * m), bh16 = (_Float16)(bv[g] * m);
        const h2 s2 = {sh16, sh16}, b2 = {bh16, bh16};
        S.sb[g][tid] = make_uint2(__builtin_bit_cast(uint32_t, s2), __builtin_bit_cast(uint32_t, b2));
      }
      S.wsh[tid] = int8_t(wsh);
      flag |= wsh;
    }
    return flag;
  };

  // fp16 exponent of 1024 in both halves (4-bit), or in every byte (8-bit),
  // kept in a register (see q4_word_to_f16 and q8_words_to_f16)
  uint32_t magic = QB == 8 ? 0x64646464u : 0x64006400u;
  asm volatile("" : "+v"(magic));
  f32x4 acc[kNT][RB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[nt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  // A slab that carries exponents: the accumulators are brought to the slab's
  // scale (times 2^-(h exponent + weight exponent) of each output) before its
  // steps accumulate, and back after, both exact.
  auto rescale = [&](const Slab<RB, GPS> &S, int sign) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int ash = GATEUP ? 0 : int(S.ash[rb * 16 + lr]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[nt][rb][i] *= pow2(sign * (ash + S.wsh[(wave * kNT + nt) * 16 + lg * 4 + i]));
    }
  };

  // One slab of every tile of this wave, in kSteps MFMA steps, for the first
  // NRB row blocks.  Row blocks past the tile's rows but below NRB are
  // multiplied too (their results are never stored), which keeps the body
  // free of branches.
  auto compute_slab = [&](const Slab<RB, GPS> &S, const WSlab<QB> &ws, auto nrb_tag, auto fast_tag) {
    constexpr int NRB = decltype(nrb_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value;
    if constexpr (AFF && FAST) {
      // round(s*(q - z) + delta) per weight (the rest of each weight was
      // added by bias_term)
      constexpr float kOff = QB == 8 ? -1152.0f : -1032.0f;  // -(1024 + z), exact in fp16
      const h2 moff = {(_Float16)kOff, (_Float16)kOff};
      h2 s2[kNT], n2[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const _Float16 sv = __builtin_bit_cast(_Float16, uint16_t(ws.s[nt]));
        s2[nt] = h2{sv, sv};
        n2[nt] = s2[nt] * moff;
      }
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        f16x8 bx[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          bx[rb] = *reinterpret_cast<const f16x8 *>(&S.a[rb * 16 + lr][lg * 32 + j * 8]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          f16x8 aw;
          if constexpr (QB == 4) {
            const uint4 &q = ws.w[nt][0];
            const uint32_t wd = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
            aw = q4_word_to_f16_c(wd, s2[nt], n2[nt], magic);
          } else {
            const uint4 &q = ws.w[nt][j >> 1];
            aw = (j & 1) ? q8_words_to_f16_c(q.z, q.w, s2[nt], n2[nt], magic)
                         : q8_words_to_f16_c(q.x, q.y, s2[nt], n2[nt], magic);
          }
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[nt][rb] = mfma_f16(aw, bx[rb], acc[nt][rb]);
        }
      }
    } else if constexpr (AFF) {
      const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
      h2 s2[kNT], s2_16[kNT], b2[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const uint2 v = S.sb[lg / kLPG][(wave * kNT + nt) * 16 + lr];
        s2[nt] = __builtin_bit_cast(h2, v.x);
        s2_16[nt] = s2[nt] * sixteenth;
        b2[nt] = __builtin_bit_cast(h2, v.y);
      }
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        f16x8 bx[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          bx[rb] = *reinterpret_cast<const f16x8 *>(&S.a[rb * 16 + lr][lg * 32 + j * 8]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          f16x8 aw;
          if constexpr (QB == 4) {
            const uint4 &q = ws.w[nt][0];
            const uint32_t wd = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
            aw = q4_word_to_f16(wd, s2[nt], s2_16[nt], b2[nt], magic);
          } else {
            const uint4 &q = ws.w[nt][j >> 1];  // step j: words 2j, 2j+1 of the lane's 8
            aw = (j & 1) ? q8_words_to_f16(q.z, q.w, s2[nt], b2[nt], magic)
                         : q8_words_to_f16(q.x, q.y, s2[nt], b2[nt], magic);
          }
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[nt][rb] = mfma_f16(aw, bx[rb], acc[nt][rb]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        uint4 bx[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          bx[rb] = *reinterpret_cast<const uint4 *>(&S.a[rb * 16 + lr][lg * 32 + j * 8]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            if constexpr (QB == kDenseF16)
              acc[nt][rb] = mfma_f16(__builtin_bit_cast(f16x8, ws.w[nt][j]), __builtin_bit_cast(f16x8, bx[rb]),
                                     acc[nt][rb]);
            else
              acc[nt][rb] = mfma_bf16(__builtin_bit_cast(bf16x8, ws.w[nt][j]), __builtin_bit_cast(bf16x8, bx[rb]),
                                      acc[nt][rb]);
          }
        }
      }
    }
  };

  // ---- pipelined main loop ----
  // Weights run PDS slabs ahead in a ring of register buffers (two slabs for
  // 4-bit weights; 8-bit and dense slabs are two and four times larger, so
  // one); the activation slab s+1 is loaded before slab s is multiplied and
  // written to the other LDS buffer after it, behind one barrier per slab.
  // Steps past the last slab only keep the barrier pattern; their loads are
  // clamped repeats.  SLOW = true: the barrier also votes on whether the
  // next slab carries exponents, and such slabs are rescaled.  SLOW = false:
  // no rescaling; for 64-row tiles each thread notes whether a slab it
  // staged carries exponents and one vote after the last slab reports
  // whether any did (the tile's results are then discarded); 16-row tiles
  // vote at every barrier and give up at the first such slab (fewer
  // registers live across the loop: three waves per SIMD).
  // The fast path's group term, added to the (zero) accumulators before the
  // slabs: for every output (weight row n, token row m) the sum over groups g
  // of c_g(n) X_g(m), c_g = b - 1024 s - n2 the part of the group's weights
  // left out of the expansion and X_g the group sum of the staged token row,
  // as one fp16 matrix-core product of c_g * group (packed) with X_g / group
  // (the x group sums), both rounded once to fp16.
  auto bias_term = [&]() {
    int btok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int m = rb * 16 + lr;
      int tk = 0;  // rows past the tile read token 0 (never stored)
      if (m < tile.rows) {
        const int q = tile.row0 + m;
        const int t = q < a.N ? a.row_map[q] : (q - a.N) % a.T;
        tk = unsigned(t) < unsigned(a.T) ? t : 0;
      }
      btok[rb] = tk;
    }
    const int gp = a.gp;
    for (int c = 0; c < gp; c += 32) {
      // every load of the chunk first (one memory round trip), then the products
      f16x8 xb[RB], av[kNT];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        xb[rb] = *reinterpret_cast<const f16x8 *>(a.xg + int64_t(btok[rb]) * gp + c + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const bool second = GATEUP && !a.fused && nt >= NTH;
        av[nt] = *reinterpret_cast<const f16x8 *>((second ? a.bp1 : a.bp0) + (int64_t(ptile[nt]) * 16 + lr) * gp +
                                                  c + 8 * lg);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[nt][rb] = mfma_f16(av[nt], xb[rb], acc[nt][rb]);
    }
  };

  constexpr int PDS = QB == 4 ? 2 : 1;
  constexpr bool kLateVote = RB > 1;
  auto run = [&](auto slow_tag, auto nrb_tag, auto fast_tag) __attribute__((always_inline)) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value;  // no exponents: no votes
    constexpr bool VOTE = !FAST && (SLOW || !kLateVote);  // vote at every barrier
    WSlab<QB> wb[PDS];
    auto load_w = [&](int s, WSlab<QB> &dst) {
      if constexpr (FAST) load_slab_fast(s, dst);
      else load_slab(s, dst);
    };
    stage_load(0, fast_tag);
    int flag;
    if constexpr (FAST) {
#pragma unroll
      for (int u = 0; u < PDS; ++u) load_w(u, wb[u]);
      bias_term();
      flag = stage_write(0, fast_tag);
    } else {
      flag = stage_write(0, fast_tag);
#pragma unroll
      for (int u = 0; u < PDS; ++u) load_w(u, wb[u]);
    }
    if constexpr (VOTE) flag = __syncthreads_or(flag);
    else __syncthreads();
    if (!SLOW && VOTE && flag) return true;
    for (int s0 = 0; s0 < nslab; s0 += PDS) {
#pragma unroll
      for (int u = 0; u < PDS; ++u) {
        const int s = s0 + u, buf = s & 1;
        stage_load(s + 1, fast_tag);
        if (SLOW && flag && col_ok) rescale(sm[buf], -1);
        if (col_ok && s < nslab) compute_slab(sm[buf], wb[u], nrb_tag, fast_tag);
        load_w(s + PDS, wb[u]);
        if (SLOW && flag && col_ok) rescale(sm[buf], +1);
        if constexpr (VOTE) {
          flag = __syncthreads_or(stage_write(buf ^ 1, fast_tag));
          if (!SLOW && flag) return true;
        } else {
          flag |= stage_write(buf ^ 1, fast_tag);
          __syncthreads();
        }
      }
    }
    if constexpr (VOTE || !AFF || FAST) return false;
    else return __syncthreads_or(flag) != 0;
  };
  // The fast loop multiplies only the row blocks that hold rows of the tile
  // (one loop per count for 64-row tiles); the rescaling loop all of them.
  // 4-bit down with groups of 32 keeps one loop: with four it no longer fits
  // its registers.
  using Full = std::integral_constant<int, RB>;
  constexpr bool kPerCount = RB == 4 && !(QB == 4 && GPS == 4 && !GATEUP);
  auto run_counts = [&](auto fast_tag) -> bool {
    if constexpr (kPerCount) {
      const int nrb = min(RB, (tile.rows + 15) / 16);
      if (nrb == 4) return run(std::false_type{}, Full{}, fast_tag);
      if (nrb == 3) return run(std::false_type{}, std::integral_constant<int, 3>{}, fast_tag);
      if (nrb == 2) return run(std::false_type{}, std::integral_constant<int, 2>{}, fast_tag);
      return run(std::false_type{}, std::integral_constant<int, 1>{}, fast_tag);
    } else {
      return run(std::false_type{}, Full{}, fast_tag);
    }
  };
  bool redo = false;
  if constexpr (AFF && GATEUP) {
    if (fast) run_counts(std::true_type{});
    else redo = run_counts(std::false_type{});
  } else {
    redo = run_counts(std::false_type{});
  }
  if (redo) {
    if constexpr (AFF) {
      // Every wave left the fast loop at the same vote, after its last read
      // of the slab buffers.
      zero_acc();
      run(std::true_type{}, Full{}, std::false_type{});
    }
  }

  if constexpr (RAW) {
    // gate and up values (the token exponent undone) as fp32: row r holds
    // gate columns 0..n_out-1 then up columns n_out..2*n_out-1
    if (!col_ok) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int m = rb * 16 + lr;
      if (m >= tile.rows) continue;
      const float xs = AFF ? pow2(rsh[m]) : 1.0f;
      float *orow = static_cast<float *>(a.out) + (tile.row0 + m) * int64_t(2 * a.n_out);
#pragma unroll
      for (int nt = 0; nt < NTH; ++nt) {
        const int c = col0 + nt * 16 + lg * 4;
        *reinterpret_cast<float4 *>(orow + c) = make_float4(acc[nt][rb][0] * xs, acc[nt][rb][1] * xs,
                                                            acc[nt][rb][2] * xs, acc[nt][rb][3] * xs);
        *reinterpret_cast<float4 *>(orow + a.n_out + c) =
            make_float4(acc[nt + NTH][rb][0] * xs, acc[nt + NTH][rb][1] * xs, acc[nt + NTH][rb][2] * xs,
                        acc[nt + NTH][rb][3] * xs);
      }
    }
    return;
  } else if constexpr (GATEUP && AFF) {
    // The GLU on the true gate/up values (the token exponent undone), then h as
    // fp16 with one exponent per (row, this block's 128 columns), in the
    // permuted staging order.  Lane (lr, lg) holds columns c..c+3,
    // c = col0 + nt*16 + 4*lg, of row m = rb*16 + lr: the lanes lg and lg^1
    // hold the two halves of an 8-column block and swap a pair of values so
    // that each stores 4 contiguous permuted elements.
    float hv[RB][NTH][4];
    with_glu(a.round_ops, a.geglu != 0, [&](auto mode, auto gelu) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb * 16 >= tile.rows) break;  // row blocks past the tile (uniform)
        const float xs = pow2(rsh[rb * 16 + lr]);
        float mx = 0.f;
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = glu_t<decltype(mode)::value, decltype(gelu)::value>(acc[nt][rb][i] * xs,
                                                                              acc[nt + NTH][rb][i] * xs);
            hv[rb][nt][i] = col_ok ? v : 0.f;
            mx = fmaxf(mx, fabsf(hv[rb][nt][i]));
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (lg == 0) rmax[wave][rb * 16 + lr] = mx;
      }
    });
    __syncthreads();
    if (!col_ok) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb * 16 >= tile.rows) break;
      const int m = rb * 16 + lr;
      float mx = rmax[0][m];
#pragma unroll
      for (int w = 1; w < kNW; ++w) mx = fmaxf(mx, rmax[w][m]);
      const int sh = f16_shift(mx);
      const float sc = pow2(-sh);
      const int64_t row = tile.row0 + m;
#pragma unroll
      for (int nt = 0; nt < NTH; ++nt) {
        const h2 v01 = {(_Float16)(hv[rb][nt][0] * sc), (_Float16)(hv[rb][nt][1] * sc)};
        const h2 v23 = {(_Float16)(hv[rb][nt][2] * sc), (_Float16)(hv[rb][nt][3] * sc)};
        const uint32_t u01 = __builtin_bit_cast(uint32_t, v01), u23 = __builtin_bit_cast(uint32_t, v23);
        const bool hi = lg & 1;  // this lane holds elements 4..7 of the block
        const uint32_t recv = __shfl_xor(hi ? u01 : u23, 16, kWave);
        uint2 o;
        if (!hi) {  // e0,e4,e1,e5 (recv = e4,e5)
          o.x = (u01 & 0xffffu) | (recv << 16);
          o.y = (u01 >> 16) | (recv & 0xffff0000u);
        } else {    // e2,e6,e3,e7 (recv = e2,e3; own e4,e5 | e6,e7)
          o.x = (recv & 0xffffu) | (u23 << 16);
          o.y = (recv >> 16) | (u23 & 0xffff0000u);
        }
        const int c = col0 + nt * 16 + lg * 4;
        if (m < tile.rows) *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) = o;
      }
      if (wave == 0 && lg == 0 && m < tile.rows) a.out_sh[row * a.nblk + bx] = int8_t(sh);
    }
    return;
  }
  if (!col_ok) return;

  // Epilogue: lane holds outputs n = col + lg*4 + i of tile row m = rb*16 + lr.
  // down with fp16 outputs: one exponent per (row, this wave's 64 columns),
  // from the row's largest magnitude over the four lanes lg that hold it.
  int ysh[RB] = {};
  if constexpr (!GATEUP) {
    static_assert(kNT * 16 == kYsBlock, "a wave writes one exponent block of each row");
    if (a.out_sh) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = 0.f;
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[nt][rb][i]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        ysh[rb] = f16_shift(mx);
        const int m = rb * 16 + lr;
        if (lg == 0 && m < tile.rows)
          a.out_sh[(tile.row0 + m) * (a.n_out / kYsBlock) + col0 / kYsBlock] = int8_t(ysh[rb]);
      }
    }
  }
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
        for (int i = 0; i < 4; ++i) {
          const float v = glu(acc[nt][rb][i], acc[nt + NTH][rb][i], a.round_ops, a.geglu);
          hb[i] = QB == kDenseF16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
        }
        const uint2 o = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) = o;
      } else if (a.out_sh) {
        const float sc = pow2(-ysh[rb]);
        const h2 v01 = {(_Float16)(acc[nt][rb][0] * sc), (_Float16)(acc[nt][rb][1] * sc)};
        const h2 v23 = {(_Float16)(acc[nt][rb][2] * sc), (_Float16)(acc[nt][rb][3] * sc)};
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) =
            make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + z * a.part_stride + row * a.n_out + c) =
            make_float4(acc[nt][rb][0], acc[nt][rb][1], acc[nt][rb][2], acc[nt][rb][3]);
      }
    }
  }
}

// Two entry points over the same body.  The second asks for two waves per
// SIMD, so that the register allocator keeps the 64-row tiles within 256
// registers (accumulators included) without spilling; left to itself it
// gives them one wave per SIMD and moves the accumulators between register
// files every slab.  16-row tiles allocate on their own.
template <int MODE, int QB, int RB, int GPS>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs a) {
  grouped_gemm_body<MODE, QB, RB, GPS>(a);
}
template <int MODE, int QB, int RB, int GPS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void grouped_gemm_kernel_w2(
    GemmArgs a) {
  grouped_gemm_body<MODE, QB, RB, GPS>(a);
}

// ---- down projection with the tile's h rows resident in LDS ---------------
// When a tile's h rows fit in LDS whole (the down reduction is d_ff), one
// workgroup stages them once and then runs several 256-column blocks of the
// output over them: the weights stream through a register ring two slabs
// ahead across column-block boundaries, each lane loads its own scales, and
// the main loop has no barrier.  (The slab-pipelined kernel above stages the
// same h rows again for every column block, with a barrier per slab.)
// Exponents: the h rows carry one per (row, 128 columns), the weights one
// per (row, slab) from |s|*qmax + |b| of the lane's group; a ballot finds the
// usual case where all are zero, otherwise the accumulators are brought to
// the slab's scale and back as in the slab-pipelined kernel (exact).
constexpr int kResMaxLds = 80 * 1024;  // bytes of resident h per workgroup

template <int QB, int RB, int GPS>
__device__ __forceinline__ void down_resident_body(const GemmArgs &a, int cbpw) {
  constexpr int NT = kNT;                   // 16-row weight tiles per wave (64 output columns)
  constexpr int PDS = (QB == 8 && RB == 4) ? 1 : 2;  // weight slabs in flight ahead (8-bit 64-row: registers)
  constexpr int NR = PDS + 1;               // ring size
  constexpr float kQMax = QB == 8 ? 255.0f : 15.0f;
  extern __shared__ __align__(16) uint16_t hs[];  // [RB*16][XR] h rows, then [RB*16][nslab] int8 exponents

  const int n_cb = (a.n_out + kNRows - 1) / kNRows;
  const int nbx = gridDim.x, total = nbx * gridDim.y;
  const int n_tiles = a.counters[1];
  const int work = n_tiles * nbx;
  const int lin = blockIdx.y * nbx + blockIdx.x;
  const int per = (work + 7) / 8;
  int item = lin;
  if (8 * per <= total) {
    const int slot = lin / 8;
    if (slot >= per) return;
    item = (lin % 8) * per + slot;
  }
  if (item >= work) return;
  int tile_id, grp;
  item_tile_block(item, n_tiles, nbx, col_group(a, nbx), tile_id, grp);
  PlanItem tile = a.tiles[tile_id];
  tile.expert = __builtin_amdgcn_readfirstlane(tile.expert);
  tile.row0 = __builtin_amdgcn_readfirstlane(tile.row0);
  tile.rows = __builtin_amdgcn_readfirstlane(tile.rows);
  const int cb0 = grp * cbpw, ncb = min(cbpw, n_cb - cb0);

  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, KW = K * QB / 32, G = K / (kKS / GPS);
  const int nslab = (K + kKS - 1) / kKS, KR = nslab * kKS, XR = KR + 8;
  int8_t *ash = reinterpret_cast<int8_t *>(hs + RB * 16 * XR);

  // ---- h rows of the tile (already fp16 in the staging order) and their exponents
  int hflag = 0;
  {
    const int P = KR / 8;  // 16-byte pieces per LDS row
    for (int q = tid; q < RB * 16 * P; q += kThreads) {
      const int m = q / P, pc = q % P;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < tile.rows && pc * 8 < K)
        v = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + int64_t(tile.row0 + m) * K)[pc];
      *reinterpret_cast<uint4 *>(&hs[m * XR + pc * 8]) = v;
    }
    for (int q = tid; q < RB * 16 * nslab; q += kThreads) {
      const int m = q / nslab, sl = q % nslab;
      const int e = m < tile.rows ? a.act_sh[int64_t(tile.row0 + m) * a.nblk + sl] : 0;
      ash[q] = int8_t(e);
      hflag |= e;
    }
  }
  hflag = __syncthreads_or(hflag);

  // ---- weights: step q = (column block j = q / nslab, slab s = q % nslab)
  const int Q = ncb * nslab;
  struct WStep {
    uint4 w[NT][QB / 4];
    uint16_t sv[NT], bv[NT];
  };
  const uint32_t *wbase = static_cast<const uint32_t *>(a.w0) + int64_t(tile.expert) * a.n_out * KW;
  // tile-packed copy (or null): the 16 rows of a slab in one block
  constexpr int SW = kKS * QB / 32;
  const uint32_t *pbase = a.wp0 ? a.wp0 + int64_t(tile.expert) * a.n_out * nslab * SW : nullptr;
  const uint16_t *sbase = a.s0 + int64_t(tile.expert) * G * a.n_out;
  const uint16_t *bbase = a.b0 + int64_t(tile.expert) * G * a.n_out;
  auto load_step = [&](int q, WStep &st) {
    q = min(q, Q - 1);
    const int j = q / nslab, sl = q % nslab;
    const int colw = (cb0 + j) * kNRows + wave * NT * 16;  // first column of this wave
    const int w = min(sl * (kKS * QB / 32) + lg * QB, KW - QB);
    const int gl = (sl * kKS + lg * 32) / (kKS / GPS);
    const int g = min(gl, G - 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = min(colw + nt * 16 + lr, a.n_out - 1);
      const uint32_t *wr = pbase ? pbase + (int64_t(n >> 4) * nslab + sl) * 16 * SW + (n & 15) * SW + lg * QB
                                 : wbase + int64_t(n) * KW + w;
#pragma unroll
      for (int v = 0; v < QB / 4; ++v) st.w[nt][v] = *reinterpret_cast<const uint4 *>(wr + 4 * v);
      const uint16_t s = sbase[int64_t(g) * a.n_out + n], b = bbase[int64_t(g) * a.n_out + n];
      st.sv[nt] = gl < G ? s : uint16_t(0);
      st.bv[nt] = gl < G ? b : uint16_t(0);
    }
  };

  uint32_t magic = QB == 8 ? 0x64646464u : 0x64006400u;
  asm volatile("" : "+v"(magic));
  f32x4 acc[NT][RB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[nt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  auto epilogue = [&](int j) {
    const int col0 = (cb0 + j) * kNRows + wave * NT * 16;
    if (col0 >= a.n_out) return;
    int ysh[RB] = {};
    if (a.out_sh) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[nt][rb][i]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        ysh[rb] = f16_shift(mx);
        const int m = rb * 16 + lr;
        if (lg == 0 && m < tile.rows)
          a.out_sh[(tile.row0 + m) * (a.n_out / kYsBlock) + col0 / kYsBlock] = int8_t(ysh[rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int m = rb * 16 + lr;
      if (m >= tile.rows) continue;
      const int64_t row = tile.row0 + m;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + nt * 16 + lg * 4;
        if (a.out_sh) {
          const float sc = pow2(-ysh[rb]);
          const h2 v01 = {(_Float16)(acc[nt][rb][0] * sc), (_Float16)(acc[nt][rb][1] * sc)};
          const h2 v23 = {(_Float16)(acc[nt][rb][2] * sc), (_Float16)(acc[nt][rb][3] * sc)};
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + c) =
              make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
        } else {
          *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * a.n_out + c) =
              make_float4(acc[nt][rb][0], acc[nt][rb][1], acc[nt][rb][2], acc[nt][rb][3]);
        }
      }
    }
  };

  // One step's MFMAs over the first NRB row blocks.
  auto compute = [&](const WStep &st, int q, auto nrb_tag) {
    constexpr int NRB = decltype(nrb_tag)::value;
    const int sl = q % nslab;
    float sv[NT], bv[NT];
    bool need = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sv[nt] = a.half_f16 ? f16_bits_to_f32(st.sv[nt]) : bf16_bits_to_f32(st.sv[nt]);
      bv[nt] = a.half_f16 ? f16_bits_to_f32(st.bv[nt]) : bf16_bits_to_f32(st.bv[nt]);
      need |= f16_shift(__builtin_fmaf(kQMax, fabsf(sv[nt]), fabsf(bv[nt]))) != 0;
    }
    const bool wexp = __ballot(need) != 0;  // uniform
    int wsh[NT] = {};
    if (wexp) {
      // the exponent of each weight row over its four lanes lg
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float wm = __builtin_fmaf(kQMax, fabsf(sv[nt]), fabsf(bv[nt]));
        wm = fmaxf(wm, __shfl_xor(wm, 16, kWave));
        wm = fmaxf(wm, __shfl_xor(wm, 32, kWave));
        wsh[nt] = f16_shift(wm);
      }
    }
    const bool rescale = wexp || hflag;
    auto scale_acc = [&](int sign) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int hsh = ash[(rb * 16 + lr) * nslab + sl];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[nt][rb][i] *= pow2(sign * (hsh + __shfl(wsh[nt], 4 * lg + i, kWave)));
      }
    };
    if (rescale) scale_acc(-1);
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    h2 s2[NT], s2_16[NT], b2[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float m = pow2(-wsh[nt]);
      const _Float16 s16 = (_Float16)(sv[nt] * m), b16 = (_Float16)(bv[nt] * m);
      s2[nt] = h2{s16, s16};
      b2[nt] = h2{b16, b16};
      s2_16[nt] = s2[nt] * sixteenth;
    }
    const uint16_t *hrow = hs + sl * kKS + lg * 32;
#pragma unroll
    for (int jj = 0; jj < kSteps; ++jj) {
      f16x8 bx[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) bx[rb] = *reinterpret_cast<const f16x8 *>(hrow + (rb * 16 + lr) * XR + jj * 8);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x8 aw;
        if constexpr (QB == 4) {
          const uint4 &qv = st.w[nt][0];
          aw = q4_word_to_f16(jj == 0 ? qv.x : jj == 1 ? qv.y : jj == 2 ? qv.z : qv.w, s2[nt], s2_16[nt], b2[nt],
                              magic);
        } else {
          const uint4 &qv = st.w[nt][jj >> 1];
          aw = (jj & 1) ? q8_words_to_f16(qv.z, qv.w, s2[nt], b2[nt], magic)
                        : q8_words_to_f16(qv.x, qv.y, s2[nt], b2[nt], magic);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[nt][rb] = mfma_f16(aw, bx[rb], acc[nt][rb]);
      }
    }
    if (rescale) scale_acc(+1);
  };

  auto run = [&](auto nrb_tag) {
    WStep ring[NR];
#pragma unroll
    for (int u = 0; u < PDS; ++u) load_step(u, ring[u]);
    for (int q0 = 0; q0 < Q; q0 += NR) {
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int q = q0 + u;
        if (q < Q) {
          load_step(q + PDS, ring[(u + PDS) % NR]);
          compute(ring[u], q, nrb_tag);
          if (q % nslab == nslab - 1) {
            epilogue(q / nslab);
            zero_acc();
          }
        }
      }
    }
  };
  const int nrb = min(RB, (tile.rows + 15) / 16);
  if constexpr (RB == 4) {
    if (nrb == 4) run(std::integral_constant<int, 4>{});
    else if (nrb == 3) run(std::integral_constant<int, 3>{});
    else if (nrb == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, RB>{});
  }
}
// 64-row tiles ask for two waves per SIMD (accumulators and the weight ring
// within 256 registers); 16-row tiles allocate on their own.
template <int QB, int RB, int GPS>
__global__ __launch_bounds__(kThreads) void down_resident_kernel(GemmArgs a, int cbpw) {
  down_resident_body<QB, RB, GPS>(a, cbpw);
}
template <int QB, int RB, int GPS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_resident_kernel_w2(
    GemmArgs a, int cbpw) {
  down_resident_body<QB, RB, GPS>(a, cbpw);
}

// ---- decode tiles (at most 16 rows of an expert, K <= 2048) ----------------
// One wave owns 16 weight rows and loads all of their codes and scales at
// once (one memory round trip), while the workgroup stages the tile's
// activation rows in LDS once; then the wave runs its K/32 MFMA steps with
// no further barrier.  Exponents are per row over the whole K (weights: the
// row's largest qmax|s| + |b|; activations: the token's x exponent, or the h
// row's largest value), so they are undone once in the epilogue.
// gate/up: a wave's rows are 8 gate rows and the 8 up rows of the same
// columns (the GLU pairs sit 32 lanes apart in the MFMA result), h is
// written as bf16.  down: 16 output columns, h read as bf16.
constexpr int kDecMaxK = 2048;  // 16 slabs: 64 (4-bit) or 128 (8-bit) registers of codes per lane

struct DecArgs {
  const void *act;          // gate/up: fp16 staging copy of x [T][K]; down: h bf16 [rows][K]
  const int8_t *act_sh;     // gate/up: token exponents [T]
  const int32_t *row_map;   // gate/up only
  int T, N, K, n_out, fused, round_ops, geglu, gsize;
  int half_f16;             // scales/biases are fp16 (else bf16)
  const uint32_t *w0;       // gate (or gate_up) / down codes
  const uint16_t *s0, *b0;
  const uint32_t *w1;       // up codes (separate layout)
  const uint16_t *s1, *b1;
  const int32_t *counters;
  const PlanItem *tiles;
  void *out;                // gate/up: h bf16 [rows][F]; down: y fp32 [rows][D]
};

template <bool GATEUP, int QB, int kMaxSlabs>
__global__ __launch_bounds__(kThreads) void decode_gemm_kernel(DecArgs a) {
  constexpr float kQMax = QB == 8 ? 255.0f : 15.0f;
  constexpr int WPL = QB;  // code words per lane and slab
  constexpr int CPW = GATEUP ? 8 : 16;           // output columns per wave
  extern __shared__ uint16_t xs[];               // [16][K + 8] activation rows, fp16 staging order
  __shared__ uint32_t rmax_bits[16];             // down: row maxima of |h| (as float bits)

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
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, KW = K * QB / 32, G = K / a.gsize, nslab = (K + kKS - 1) / kKS;
  // LDS rows hold whole slabs (K rounded up to 128, the tail zeroed) plus a
  // pad that spreads the 16 rows over banks.
  const int KR = nslab * kKS, XR = KR + 8;
  const int col0 = (bx * kNW + wave) * CPW;
  const bool col_ok = col0 < a.n_out;
  const int colc = col_ok ? col0 : a.n_out - CPW;

  // ---- this lane's weight row: codes and scales for the whole K ----
  const bool up = GATEUP && lr >= 8;
  const int rcol = colc + (GATEUP ? (lr & 7) : lr);
  const int nre = (GATEUP && a.fused) ? 2 * a.n_out : a.n_out;  // rows of one expert's matrix
  const int rin = (GATEUP && a.fused && up ? a.n_out : 0) + rcol;
  const bool second = GATEUP && !a.fused && up;
  const uint32_t *wrow = (second ? a.w1 : a.w0) + (int64_t(tile.expert) * nre + rin) * KW;
  const uint16_t *sp = (second ? a.s1 : a.s0) + int64_t(tile.expert) * G * nre + rin;
  const uint16_t *bp = (second ? a.b1 : a.b0) + int64_t(tile.expert) * G * nre + rin;
  uint4 wq[kMaxSlabs][QB / 4];
  uint16_t sr[kMaxSlabs], br[kMaxSlabs];
#pragma unroll
  for (int s = 0; s < kMaxSlabs; ++s) {
    const int sc = min(s, nslab - 1);
    const int w = min(sc * (kKS * QB / 32) + lg * WPL, KW - WPL);
#pragma unroll
    for (int v = 0; v < QB / 4; ++v) wq[s][v] = *reinterpret_cast<const uint4 *>(wrow + w + 4 * v);
    // this lane's 32 elements of the slab lie in one group
    const int gl = (sc * kKS + lg * 32) / a.gsize;
    const int g = min(gl, G - 1);
    const bool ok = s < nslab && gl < G;
    const uint16_t sv = sp[int64_t(g) * nre], bv = bp[int64_t(g) * nre];
    sr[s] = ok ? sv : uint16_t(0);
    br[s] = ok ? bv : uint16_t(0);
  }

  // ---- stage the tile's activation rows (fp16 staging order) ----
  const int P = K / 8;  // 16-byte pieces per row
  if (tid < 16) rmax_bits[tid] = 0u;
  for (int q = tid; q < 16 * (KR - K) / 8; q += kThreads) {
    const int nz = (KR - K) / 8;
    *reinterpret_cast<uint4 *>(&xs[(q / nz) * XR + K + (q % nz) * 8]) = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // Only the tile's own rows are staged: MFMA result column m depends only
  // on activation row m, and the columns of rows past the tile are never
  // stored, whatever those LDS rows hold.
  const int nrow = min(tile.rows, 16);
  if constexpr (GATEUP) {
    for (int q = tid; q < nrow * P; q += kThreads) {
      const int m = q / P, pc = q % P;
      const int p = tile.row0 + m;
      const int tok = p < a.N ? a.row_map[p] : (p - a.N) % a.T;
      const int tk = unsigned(tok) < unsigned(a.T) ? tok : 0;
      *reinterpret_cast<uint4 *>(&xs[m * XR + pc * 8]) =
          reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + int64_t(tk) * K)[pc];
    }
  } else {
    // h rows (bf16): row maxima first, then fp16 with one exponent per row
    // (the second pass re-reads the rows, now in cache)
    for (int q0 = 0; q0 < nrow * P; q0 += 4 * kThreads) {
      uint4 hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = min(q0 + tid + i * kThreads, nrow * P - 1);
        const int m = q / P, pc = q % P;
        const int p = tile.row0 + m;
        hv[i] = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + int64_t(p) * K)[pc];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + tid + i * kThreads;
        if (q < nrow * P) atomicMax(&rmax_bits[q / P], __float_as_uint(absmax8(hv[i], false)));
      }
    }
    __syncthreads();
    for (int q = tid; q < nrow * P; q += kThreads) {
      const int m = q / P, pc = q % P;
      const int p = tile.row0 + m;
      const uint4 v = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + int64_t(p) * K)[pc];
      *reinterpret_cast<uint4 *>(&xs[m * XR + pc * 8]) =
          permute8(half8_to_f16(v, f16_shift(__uint_as_float(rmax_bits[m])), false));
    }
  }

  // ---- weight row exponent over the whole K, fp16 scales ----
  float sf[kMaxSlabs], bf[kMaxSlabs], wm = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSlabs; ++s) {
    sf[s] = a.half_f16 ? f16_bits_to_f32(sr[s]) : bf16_bits_to_f32(sr[s]);
    bf[s] = a.half_f16 ? f16_bits_to_f32(br[s]) : bf16_bits_to_f32(br[s]);
    wm = fmaxf(wm, __builtin_fmaf(kQMax, fabsf(sf[s]), fabsf(bf[s])));
  }
  wm = fmaxf(wm, __shfl_xor(wm, 16, kWave));
  wm = fmaxf(wm, __shfl_xor(wm, 32, kWave));
  const int wsh = f16_shift(wm);  // exponent of weight row lr
  const float wmul = pow2(-wsh);
  __syncthreads();  // activation rows staged

  uint32_t magic = QB == 8 ? 0x64646464u : 0x64006400u;
  asm volatile("" : "+v"(magic));
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSlabs; ++s) {
    if (s < nslab) {
      const _Float16 s16 = (_Float16)(sf[s] * wmul), b16 = (_Float16)(bf[s] * wmul);
      const h2 s2 = {s16, s16}, b2 = {b16, b16};
      const h2 s2_16 = s2 * sixteenth;
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        const f16x8 bxv = *reinterpret_cast<const f16x8 *>(&xs[lr * XR + s * kKS + lg * 32 + j * 8]);
        f16x8 aw;
        if constexpr (QB == 4) {
          const uint4 &q = wq[s][0];
          aw = q4_word_to_f16(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w, s2, s2_16, b2, magic);
        } else {
          const uint4 &q = wq[s][j >> 1];
          aw = (j & 1) ? q8_words_to_f16(q.z, q.w, s2, b2, magic) : q8_words_to_f16(q.x, q.y, s2, b2, magic);
        }
        acc = mfma_f16(aw, bxv, acc);
      }
    }
  }

  // ---- epilogue: lane holds weight rows 4*lg + i of token row m = lr ----
  // true value = acc * 2^(weight row exponent + activation row exponent)
  const int m = lr;
  int ash;
  if constexpr (GATEUP) {
    const int p = tile.row0 + min(m, tile.rows - 1);
    const int tok = p < a.N ? a.row_map[p] : (p - a.N) % a.T;
    ash = a.act_sh[unsigned(tok) < unsigned(a.T) ? tok : 0];
  } else {
    ash = f16_shift(__uint_as_float(rmax_bits[m]));
  }
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int we = __shfl(wsh, 4 * lg + i, kWave);  // exponent of weight row 4*lg+i (held by lane lr = 4*lg+i)
    v[i] = acc[i] * pow2(we + ash);
  }
  const int64_t row = tile.row0 + m;
  if constexpr (GATEUP) {
    float u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __shfl_xor(v[i], 32, kWave);  // up rows 8 + 4*lg + i
    if (col_ok && lg < 2 && m < tile.rows) {
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_bits(glu(v[i], u[i], a.round_ops, a.geglu));
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * a.n_out + col0 + 4 * lg) =
          make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    }
  } else if (col_ok && m < tile.rows) {
    const int c = col0 + 4 * lg;
    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * a.n_out + c) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int MODE, int QB, int RB, int GPS>
void launch_one(const GemmArgs &ga, int64_t max_tiles, hipStream_t s) {
  constexpr int NTH = MODE != kDown ? kNT / 2 : kNT;
  const int cols_per_block = kNW * NTH * 16;
  const dim3 grid((ga.n_out + cols_per_block - 1) / cols_per_block, unsigned(max_tiles), unsigned(ga.kz));
  // 16-row tiles fit two or more waves per SIMD by themselves.
  constexpr bool kFits = RB == 1;
  if constexpr (kFits) launch((grouped_gemm_kernel<MODE, QB, RB, GPS>), grid, dim3(kThreads), 0, s, ga);
  else launch((grouped_gemm_kernel_w2<MODE, QB, RB, GPS>), grid, dim3(kThreads), 0, s, ga);
}
// Code width (0: dense bf16) and groups per slab picked at run time.
template <int MODE, int RB, int QB>
void launch_groups(const GemmArgs &ga, int gsize, int64_t max_tiles, hipStream_t s) {
  if (gsize == 32) launch_one<MODE, QB, RB, 4>(ga, max_tiles, s);
  else if (gsize == 128) launch_one<MODE, QB, RB, 1>(ga, max_tiles, s);
  else launch_one<MODE, QB, RB, 2>(ga, max_tiles, s);
}
template <int MODE, int RB>
void launch_gemm(const GemmArgs &ga, int qb, int gsize, int64_t max_tiles, hipStream_t s) {
  if (qb == 4) launch_groups<MODE, RB, 4>(ga, gsize, max_tiles, s);
  else if (qb == 8) launch_groups<MODE, RB, 8>(ga, gsize, max_tiles, s);
  else if (qb == kDenseF16) launch_one<MODE, kDenseF16, RB, 1>(ga, max_tiles, s);
  else launch_one<MODE, kDenseBF16, RB, 1>(ga, max_tiles, s);
}

// Bytes of dynamic LDS of the resident-h down kernel for RB row blocks.
inline size_t down_resident_lds(int RB, int K) {
  const int nslab = (K + kKS - 1) / kKS;
  return size_t(RB) * 16 * (nslab * kKS + 8) * sizeof(uint16_t) + size_t(RB) * 16 * nslab;
}
template <int QB, int RB>
void launch_down_resident(const GemmArgs &ga, int gsize, int64_t max_tiles, int64_t est_tiles, hipStream_t s) {
  const int n_cb = (ga.n_out + kNRows - 1) / kNRows;
  // column blocks per workgroup: about two workgroups per CU over the
  // expected tiles, each staging its tile's h once (prefill: all 8 blocks,
  // 125.6 us against 128.5 us with 5 and 169.8 us with 1; 32-token decode:
  // 2 blocks, 33.5 us against 35.3 us with 1)
  const int64_t want = (est_tiles * n_cb + 511) / 512;
  const int cbpw = int(std::max<int64_t>(1, std::min<int64_t>(n_cb, want)));
  const dim3 grid((n_cb + cbpw - 1) / cbpw, unsigned(max_tiles));
  const size_t lds = down_resident_lds(RB, ga.K);
  auto go = [&](auto kern) {
    if (lds > 64 * 1024) {
      static const bool raised = [&] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   kResMaxLds) == hipSuccess;
      }();
      (void)raised;
    }
    launch(kern, grid, dim3(kThreads), lds, s, ga, cbpw);
  };
  if constexpr (RB == 1) {
    if (gsize == 32) go(down_resident_kernel<QB, RB, 4>);
    else if (gsize == 128) go(down_resident_kernel<QB, RB, 1>);
    else go(down_resident_kernel<QB, RB, 2>);
  } else {
    if (gsize == 32) go(down_resident_kernel_w2<QB, RB, 4>);
    else if (gsize == 128) go(down_resident_kernel_w2<QB, RB, 1>);
    else go(down_resident_kernel_w2<QB, RB, 2>);
  }
}

template <bool GATEUP, int QB, int MS>
void launch_decode_ms(const DecArgs &da, int64_t max_tiles, hipStream_t s) {
  constexpr int CPW = GATEUP ? 8 : 16;
  const int cols_per_block = kNW * CPW;
  const size_t lds = size_t(16) * ((da.K + kKS - 1) / kKS * kKS + 8) * sizeof(uint16_t);
  if (lds > 64 * 1024) {
    // above the default dynamic-LDS limit (gfx950 has 160 KB per CU): raise it once
    static const bool raised = [] {
      return hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_gemm_kernel<GATEUP, QB, MS>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 int(16 * (MS * kKS + 8) * sizeof(uint16_t))) == hipSuccess;
    }();
    (void)raised;
  }
  const dim3 grid((da.n_out + cols_per_block - 1) / cols_per_block, unsigned(max_tiles));
  launch((decode_gemm_kernel<GATEUP, QB, MS>), grid, dim3(kThreads), lds, s, da);
}
// K <= 1024: 8 slabs of registers; K <= 2048: 16.
template <bool GATEUP>
void launch_decode(const DecArgs &da, int qb, int64_t max_tiles, hipStream_t s) {
  const bool short_k = da.K <= 8 * kKS;
  if (qb == 8) {
    if (short_k) launch_decode_ms<GATEUP, 8, 8>(da, max_tiles, s);
    else launch_decode_ms<GATEUP, 8, 16>(da, max_tiles, s);
  } else {
    if (short_k) launch_decode_ms<GATEUP, 4, 8>(da, max_tiles, s);
    else launch_decode_ms<GATEUP, 4, 16>(da, max_tiles, s);
  }
}

}  // namespace

bool use_mfma(const moe_layer_desc *d) {
  // 16-bit activations with every reduction length a whole number of
  // 64-element groups; fp32 layers and other shapes take the dequant-GEMV
  // kernels.
  return d->act_dtype != MOE_DT_F32 && d->d_model % 64 == 0 && d->d_ff % 64 == 0;
}

// Experts with two or more row tiles on average: the work runs in groups of
// 8 column blocks with an expert's tiles together, so all but the first tile
// read the weights from L2.
static int use_bx_major(const moe_layer_desc *d, int32_t T) {
  const int64_t rows_per_expert = int64_t(T) * d->top_k / d->n_experts;
  return rows_per_expert >= 2 * plan_tile_rows(d, T) ? 1 : 0;
}

// The decode tiles: 16-row tiles of affine layers with at most one routed
// row per expert on average and both reduction lengths within kDecMaxK.
static bool decode_tiles(const moe_layer_desc *d, int32_t T) {
  return use_mfma(d) && plan_tile_rows(d, T) == 16 && affine(d) && int64_t(T) * d->top_k <= d->n_experts &&
         d->d_model <= kDecMaxK && d->d_ff <= kDecMaxK;
}

int ffn_down_parts(const moe_layer_desc *d, int32_t T) {
  // Few workgroups in the down projection (few tiles, long reduction, as in a
  // dense layer with 8 experts): split the reduction until about 512
  // workgroups, at least two slabs per part.
  if (T <= 0 || !use_mfma(d) || decode_tiles(d, T)) return 1;
  const int64_t R = int64_t(T) * d->top_k + int64_t(d->n_shared) * T;
  const int tr = plan_tile_rows(d, T);
  const int64_t tiles = std::max<int64_t>(std::min<int64_t>(R, d->n_experts + d->n_shared), (R + tr - 1) / tr);
  const int64_t nbx = (d->d_model + kNRows - 1) / kNRows;
  const int nslab = (d->d_ff + kKS - 1) / kKS;
  int kz = 1;
  while (tiles * nbx * kz < 512 && kz < 8 && nslab >= 4 * kz) kz *= 2;
  const int ns = (nslab + kz - 1) / kz;
  return (nslab + ns - 1) / ns;  // every part non-empty
}

int64_t ys_workspace_bytes(const moe_layer_desc *d, int32_t T) {
  // fp32 rows bound fp16 ones.  Partial rows: a split into p > 1 parts
  // stopped doubling with tiles * nbx * p < 1024, and R <= 64 * tiles, so
  // p * R < 1024 * 64 / nbx; p is at most the largest split the reduction
  // length allows.  Both bounds grow with T, so the size also covers every
  // smaller T.
  const int64_t R = int64_t(T) * d->top_k + int64_t(d->n_shared) * T, D = d->d_model;
  int64_t rows = R;
  if (use_mfma(d)) {
    const int nslab = (d->d_ff + kKS - 1) / kKS;
    const int64_t kzmax = nslab >= 16 ? 8 : nslab >= 8 ? 4 : nslab >= 4 ? 2 : 1;
    const int64_t nbx = (D + kNRows - 1) / kNRows;
    rows = std::max(R, std::min(kzmax * R, 1024 * 64 / nbx));
  }
  return rows * D * 4;
}

bool ys_f16e(const moe_layer_desc *d, int32_t T) {
  return use_mfma(d) && !decode_tiles(d, T) && ffn_down_parts(d, T) == 1;
}

int plan_tile_rows(const moe_layer_desc *d, int32_t T) {
  // Decode-sized groups (T*k/E <= 8 rows per expert on average, the pages'
  // small-group regime) use 16-row tiles; larger groups 64-row tiles.
  const int64_t N = int64_t(T) * d->top_k;
  return N <= 8LL * d->n_experts ? 16 : 64;
}

// The tile-packed copies, when the caller gave every one the projection
// needs (gate and up both, when separate).
// p1: the up projection when gate and up are separate, else null.
// proj0/proj1: their moe_projection values.  xg (nullable): the token group
// means (XgOut), which turn on the fast path of gate/up.
static void set_packed(const moe_layer_desc *d, GemmArgs &g, const moe_proj &p0, const moe_proj *p1, int proj0,
                       int proj1, const uint16_t *xg = nullptr) {
  if (!affine(d) || !p0.w_packed || (p1 && !p1->w_packed)) return;
  PackedLayout L0, L1;
  if (!packed_layout(d, proj0, &L0) || (p1 && !packed_layout(d, proj1, &L1))) return;
  auto at = [](const void *base, size_t off) { return static_cast<const unsigned char *>(base) + off; };
  g.wp0 = reinterpret_cast<const uint32_t *>(at(p0.w_packed, L0.codes));
  g.wp1 = p1 ? reinterpret_cast<const uint32_t *>(at(p1->w_packed, L1.codes)) : nullptr;
  if (!xg || L0.GP != xg_groups_padded(d)) return;
  g.sp0 = reinterpret_cast<const uint16_t *>(at(p0.w_packed, L0.scales));
  g.bp0 = reinterpret_cast<const uint16_t *>(at(p0.w_packed, L0.biases));
  g.fl0 = reinterpret_cast<const int32_t *>(at(p0.w_packed, L0.flags));
  if (p1) {
    g.sp1 = reinterpret_cast<const uint16_t *>(at(p1->w_packed, L1.scales));
    g.bp1 = reinterpret_cast<const uint16_t *>(at(p1->w_packed, L1.biases));
    g.fl1 = reinterpret_cast<const int32_t *>(at(p1->w_packed, L1.flags));
  }
  g.xg = xg;
  g.gp = L0.GP;
}

void launch_gate_up_raw_mfma(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                             const moe_weights *w, const int32_t *counters, const PlanItem *tiles, int64_t max_tiles,
                             const FfnScratch &sc, float *gu, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aff = affine(d);
  const bool f16 = d->act_dtype == MOE_DT_F16;
  const int qb = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : aff ? 4 : f16 ? kDenseF16 : kDenseBF16;
  if (aff && !sc.x16_ready)
    launch(act_f16_kernel, dim3((T + 3) / 4), dim3(256), 0, s, static_cast<const uint16_t *>(x), T,
                       d->d_model, static_cast<uint16_t *>(sc.x16), sc.xsh, int(f16), XgOut{nullptr, 0, 0});
  const moe_proj &pg = d->gate_up_fused ? w->gate_up : w->gate;
  GemmArgs g{aff ? sc.x16 : x, sc.xsh, nullptr, 0, row_map, T, T * d->top_k, d->d_model, d->d_ff,
             d->gate_up_fused, 0, 0, int(f16),
             pg.w, static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pg.biases),
             w->up.w, static_cast<const uint16_t *>(w->up.scales), static_cast<const uint16_t *>(w->up.biases),
             counters, tiles, gu, use_bx_major(d, T), 1, 0};
  set_packed(d, g, pg, d->gate_up_fused ? nullptr : &w->up, d->gate_up_fused ? MOE_PROJ_GATE_UP : MOE_PROJ_GATE,
             MOE_PROJ_UP);
  if (plan_tile_rows(d, T) == 16) launch_gemm<kGateUpRaw, 1>(g, qb, d->group_size, max_tiles, s);
  else launch_gemm<kGateUpRaw, 4>(g, qb, d->group_size, max_tiles, s);
}

void launch_expert_ffn_mfma(const moe_layer_desc *d, int32_t T, const void *x, const int32_t *row_map,
                            const moe_weights *w, const int32_t *counters, const PlanItem *tiles,
                            int64_t max_tiles, const FfnScratch &sc, void *y_sorted, int8_t *ys_sh, void *stream,
                            StageMarker *mk, int down_parts) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aff = affine(d);
  const bool f16 = d->act_dtype == MOE_DT_F16;
  const int qb = d->w_format == MOE_WF_AFFINE_Q8 ? 8 : aff ? 4 : f16 ? kDenseF16 : kDenseBF16;
  const int gs = d->group_size;
  const int geglu = d->activation == MOE_ACT_GEGLU;
  const int tr = plan_tile_rows(d, T);
  const int nblk = (d->d_ff + kHBlock - 1) / kHBlock;
  const int bx_major = use_bx_major(d, T);
  // the group means of x for the fast gate/up path: written with the fp16
  // staging copy, by the router (x16_ready) or here
  const XgOut xo = xg_out(d, sc.xg);
  if (aff && !sc.x16_ready) {
    launch(act_f16_kernel, dim3((T + 3) / 4), dim3(256), 0, s, static_cast<const uint16_t *>(x), T,
                       d->d_model, static_cast<uint16_t *>(sc.x16), sc.xsh, int(f16), xo);
    if (mk) mk->mark("x_f16");
  }
  const moe_proj &pg = d->gate_up_fused ? w->gate_up : w->gate;
  GemmArgs gu{aff ? sc.x16 : x, sc.xsh, sc.hsh, nblk, row_map, T, T * d->top_k, d->d_model, d->d_ff,
              d->gate_up_fused, glu_round_mode(d), geglu, int(f16),
              pg.w, static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pg.biases),
              w->up.w, static_cast<const uint16_t *>(w->up.scales), static_cast<const uint16_t *>(w->up.biases),
              counters, tiles, sc.h, bx_major, 1, 0};
  if (ys_sh && (down_parts > 1 || decode_tiles(d, T)))
    throw std::invalid_argument("expert ffn: fp16 outputs need the 64- or 16-row tiles without a reduction split");
  GemmArgs dn{sc.h, sc.hsh, ys_sh, nblk, nullptr, T, T * d->top_k, d->d_ff, d->d_model, 0, 0, 0, int(f16),
              w->down.w, static_cast<const uint16_t *>(w->down.scales), static_cast<const uint16_t *>(w->down.biases),
              nullptr, nullptr, nullptr, counters, tiles, y_sorted, bx_major, down_parts,
              (int64_t(T) * d->top_k + int64_t(d->n_shared) * T) * d->d_model};
  set_packed(d, gu, pg, d->gate_up_fused ? nullptr : &w->up, d->gate_up_fused ? MOE_PROJ_GATE_UP : MOE_PROJ_GATE,
             MOE_PROJ_UP, xo.xg);
  set_packed(d, dn, w->down, nullptr, MOE_PROJ_DOWN, MOE_PROJ_DOWN);
  if (decode_tiles(d, T)) {
    // at most one routed row per expert on average: whole-K loads per wave
    // (one memory round trip), h as bf16 between the two projections
    DecArgs dg{sc.x16, sc.xsh, row_map, T, T * d->top_k, d->d_model, d->d_ff, d->gate_up_fused,
               glu_round_mode(d), geglu, gs, int(f16), static_cast<const uint32_t *>(pg.w),
               static_cast<const uint16_t *>(pg.scales), static_cast<const uint16_t *>(pg.biases),
               static_cast<const uint32_t *>(w->up.w), static_cast<const uint16_t *>(w->up.scales),
               static_cast<const uint16_t *>(w->up.biases), counters, tiles, sc.h};
    DecArgs dd{sc.h, nullptr, nullptr, T, T * d->top_k, d->d_ff, d->d_model, 0, 0, 0, gs, int(f16),
               static_cast<const uint32_t *>(w->down.w), static_cast<const uint16_t *>(w->down.scales),
               static_cast<const uint16_t *>(w->down.biases), nullptr, nullptr, nullptr, counters, tiles, y_sorted};
    launch_decode<true>(dg, qb, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    launch_decode<false>(dd, qb, max_tiles, s);
    if (mk) mk->mark("down_mfma");
  } else {
    // the down projection keeps each tile's h rows resident in LDS when they fit
    const bool resident = aff && down_parts == 1 && down_resident_lds(tr == 16 ? 1 : 4, d->d_ff) <= kResMaxLds;
    const int64_t R = int64_t(T) * d->top_k + int64_t(d->n_shared) * T;
    const int64_t est_tiles = std::max<int64_t>(std::min<int64_t>(R, d->n_experts + d->n_shared), (R + tr - 1) / tr);
    if (tr == 16) launch_gemm<kGateUp, 1>(gu, qb, gs, max_tiles, s);
    else launch_gemm<kGateUp, 4>(gu, qb, gs, max_tiles, s);
    if (mk) mk->mark("gateup_mfma");
    if (resident && tr == 16) {
      if (qb == 8) launch_down_resident<8, 1>(dn, gs, max_tiles, est_tiles, s);
      else launch_down_resident<4, 1>(dn, gs, max_tiles, est_tiles, s);
    } else if (resident) {
      if (qb == 8) launch_down_resident<8, 4>(dn, gs, max_tiles, est_tiles, s);
      else launch_down_resident<4, 4>(dn, gs, max_tiles, est_tiles, s);
    } else if (tr == 16) {
      launch_gemm<kDown, 1>(dn, qb, gs, max_tiles, s);
    } else {
      launch_gemm<kDown, 4>(dn, qb, gs, max_tiles, s);
    }
    if (mk) mk->mark("down_mfma");
  }
}

}  // namespace moe
