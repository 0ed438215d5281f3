// f16_stage.h -- the fp16 staging format of the 4-bit matrix-core GEMMs.
//
// Activations of affine layers are multiplied as fp16.  A row is stored as
// fp16 x * 2^-e with one power-of-two exponent e per row (f16_shift), and
// every 8-element block permuted to e0,e4,e1,e5,e2,e6,e3,e7, the order in
// which the GEMMs expand eight codes.  bf16 -> fp16 is exact for values in
// fp16's normal range; fp16 rows with no exponent are copied as they are.
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 16-bit elements e0..e7 -> e0,e4,e1,e5,e2,e6,e3,e7 (the order of q4_word_to_f16).
__device__ __forceinline__ uint4 permute8(uint4 v) {
  uint4 r;
  r.x = (v.x & 0xffffu) | (v.z << 16);
  r.y = (v.x >> 16) | (v.z & 0xffff0000u);
  r.z = (v.y & 0xffffu) | (v.w << 16);
  r.w = (v.y >> 16) | (v.w & 0xffff0000u);
  return r;
}

// Power-of-two exponent e for a nonnegative magnitude, nonzero only when
// needed: mag * 2^-e lies below 2^15 (fp16 range with headroom), and
// magnitudes below 2^-10 (whose small elements would fall into fp16
// subnormals) are brought to [1, 2).  Zero needs no exponent.
__device__ __forceinline__ int f16_shift(float mag) {
  const int ex = int((__float_as_uint(mag) >> 23) & 0xffu) - 127;  // floor(log2(mag)) for normal mag
  if (ex >= 15) return ex - 14;
  if (mag > 0.f && ex < -10) return max(ex, -100);
  return 0;
}
__device__ __forceinline__ float pow2(int e) { return __uint_as_float(uint32_t(127 + e) << 23); }

// Eight 16-bit values (bf16, or fp16 when f16 is set) scaled by 2^-sh as
// packed fp16 (two per word).
template <int DT>
__device__ __forceinline__ uint4 half8_to_f16_t(uint4 v, int sh) {
  const float m = pow2(-sh);
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2_t p = {(_Float16)(half_lo<DT>(u[i]) * m), (_Float16)(half_hi<DT>(u[i]) * m)};
    o[i] = __builtin_bit_cast(uint32_t, p);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ uint4 half8_to_f16(uint4 v, int sh, bool f16) {
  if (!f16) return half8_to_f16_t<kDtBF16>(v, sh);
  return sh == 0 ? v : half8_to_f16_t<kDtF16>(v, sh);
}

template <int DT>
__device__ __forceinline__ float absmax8_t(uint4 v) {
  const float a = fmaxf(fmaxf(fabsf(half_lo<DT>(v.x)), fabsf(half_hi<DT>(v.x))),
                        fmaxf(fabsf(half_lo<DT>(v.y)), fabsf(half_hi<DT>(v.y))));
  const float b = fmaxf(fmaxf(fabsf(half_lo<DT>(v.z)), fabsf(half_hi<DT>(v.z))),
                        fmaxf(fabsf(half_lo<DT>(v.w)), fabsf(half_hi<DT>(v.w))));
  return fmaxf(a, b);
}
__device__ __forceinline__ float absmax8(uint4 v, bool f16) {
  return f16 ? absmax8_t<kDtF16>(v) : absmax8_t<kDtBF16>(v);
}

// The group means (XgOut): each group's sum in fp32 over its fp16 staged
// values, so |mean| stays within the row's largest |value|.
// Called by every lane of the wave at once: lane's piece p (8 staged values
// in any order; valid false: past the row) goes into its group's sum over the
// gs / 8 lanes that hold the group, and the group's first lane writes the mean.
__device__ __forceinline__ void group_mean_piece(uint4 o, bool valid, int p, const XgOut &xo, uint16_t *row) {
  const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float s = 0.f;
  if (valid) {
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, o.x), one2, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, o.y), one2, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, o.z), one2, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, o.w), one2, s, false);
  }
  // sums over the gs / 8 lanes of the group (4, 8 or 16; groups never
  // straddle a pass), on DPP lane moves: quads, then mirrored half rows, then
  // mirrored rows
  const int lpg = xo.gs / 8;
  s += dpp_move<kDppQuadSwap1>(0.f, s);
  s += dpp_move<kDppQuadSwap2>(0.f, s);
  if (lpg >= 8) s += dpp_move<kDppHalfMirror>(0.f, s);
  if (lpg >= 16) s += dpp_move<kDppRowMirror>(0.f, s);
  if (valid && (lane_id() & (lpg - 1)) == 0) {
    const _Float16 m = static_cast<_Float16>(s * (1.0f / float(xo.gs)));
    row[p * 8 / xo.gs] = __builtin_bit_cast(uint16_t, m);
  }
}
__device__ __forceinline__ void group_mean_pad(int D, const XgOut &xo, uint16_t *row) {
  for (int g = D / xo.gs + lane_id(); g < xo.gp; g += kWave) row[g] = 0;
}

// One wave converts row x[0..D) (bf16, or fp16 when f16 is set; D a
// multiple of 8) to out[0..D) in the staging format and writes its exponent
// to *sh_out (lane 0), and the row's group means to row t of xo when set.
__device__ __forceinline__ void row_to_f16(const uint16_t *x, int D, uint16_t *out, int8_t *sh_out, bool f16,
                                           XgOut xo = {nullptr, 0, 0}, int t = 0) {
  const int lane = lane_id();
  const uint4 *src = reinterpret_cast<const uint4 *>(x);
  uint4 *dst = reinterpret_cast<uint4 *>(out);
  const int P = D / 8;
  float mx = 0.f;
  for (int p = lane; p < P; p += kWave) mx = fmaxf(mx, absmax8(src[p], f16));
  mx = wave_max(mx);
  const int sh = f16_shift(mx);
  uint16_t *xrow = xo.xg ? xo.xg + int64_t(t) * xo.gp : nullptr;
  for (int p0 = 0; p0 < P; p0 += kWave) {  // the same trip count on every lane
    const int p = p0 + lane;
    const bool ok = p < P;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (ok) {
      o = permute8(half8_to_f16(src[p], sh, f16));
      dst[p] = o;
    }
    if (xrow) group_mean_piece(o, ok, p, xo, xrow);
  }
  if (xrow) group_mean_pad(D, xo, xrow);
  if (lane == 0) *sh_out = int8_t(sh);
}

// The same conversion split in two phases for kernels that already hold one
// wave per token (d <= 4096: at most 8 pieces of 8 per lane): row_f16_load
// issues the loads early, row_f16_store converts and stores them later.
constexpr int kRowF16MaxD = kWave * 8 * 8;
struct RowF16 {
  uint4 v[8];
};
__device__ __forceinline__ void row_f16_load(const uint16_t *x, int D, RowF16 &r) {
  const int lane = lane_id();
#pragma unroll
  for (int q = 0; q < 8; ++q) r.v[q] = reinterpret_cast<const uint4 *>(x)[min(q * kWave + lane, D / 8 - 1)];
}
__device__ __forceinline__ void row_f16_store(const RowF16 &r, int D, uint16_t *out, int8_t *sh_out, bool f16,
                                              XgOut xo = {nullptr, 0, 0}, int t = 0) {
  const int lane = lane_id();
  float mx = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if ((q * kWave + lane) * 8 < D) mx = fmaxf(mx, absmax8(r.v[q], f16));
  mx = wave_max(mx);
  const int sh = f16_shift(mx);
  uint16_t *xrow = xo.xg ? xo.xg + int64_t(t) * xo.gp : nullptr;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (q * kWave * 8 >= D) break;  // the same on every lane
    const bool ok = (q * kWave + lane) * 8 < D;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (ok) {
      o = permute8(half8_to_f16(r.v[q], sh, f16));
      reinterpret_cast<uint4 *>(out)[q * kWave + lane] = o;
    }
    if (xrow) group_mean_piece(o, ok, q * kWave + lane, xo, xrow);
  }
  if (xrow) group_mean_pad(D, xo, xrow);
  if (lane == 0) *sh_out = int8_t(sh);
}

}  // namespace moe
