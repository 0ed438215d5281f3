// device_common.h -- small device helpers for the gfx950 kernels: bf16
// conversions and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }
// The two bf16 values packed in a 32-bit word (element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.  gfx950
// converts in one instruction (v_cvt_pk_bf16_f32, under the default
// round-to-nearest-even mode, subnormals kept).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }

// Element dtypes as template arguments (the values of moe_dtype).
constexpr int kDtF32 = 0, kDtBF16 = 1, kDtF16 = 2;

// fp16 bits <-> fp32 (widening exact; narrowing rounds to nearest even).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}
__device__ __forceinline__ float f16_lo(uint32_t u) { return f16_bits_to_f32(u & 0xffffu); }
__device__ __forceinline__ float f16_hi(uint32_t u) { return f16_bits_to_f32(u >> 16); }
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, _Float16(f)); }

// A 16-bit element (DT = bf16 or fp16) as fp32; the two elements packed in a word.
template <int DT>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (DT == kDtF16) return f16_bits_to_f32(h);
  else return bf16_bits_to_f32(h);
}
template <int DT>
__device__ __forceinline__ float half_lo(uint32_t u) {
  if constexpr (DT == kDtF16) return f16_lo(u);
  else return bf16_lo(u);
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t u) {
  if constexpr (DT == kDtF16) return f16_hi(u);
  else return bf16_hi(u);
}
// fp32 -> bits of a 16-bit dtype, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t f32_to_half_bits(float f) {
  if constexpr (DT == kDtF16) return f32_to_f16_bits(f);
  else return f32_to_bf16_bits(f);
}

// Activation element i as fp32 (DT: fp32, or 16-bit bits).
template <int DT>
__device__ __forceinline__ float load_act(const void *p, int64_t i) {
  if constexpr (DT == kDtF32) return static_cast<const float *>(p)[i];
  else return half_to_f32<DT>(static_cast<const uint16_t *>(p)[i]);
}

// Wave-wide reductions on DPP lane moves (no LDS round trip): within quads,
// then mirrored half rows and rows of 16, then two row broadcasts that leave
// the result in lane 63, read back as a uniform value.  Every lane must be
// active.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_move(float old, float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
constexpr int kDppQuadSwap1 = 0xb1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4e;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppRowMirror = 0x140;  // row_mirror
constexpr int kDppBcast15 = 0x142;    // row_bcast:15
constexpr int kDppBcast31 = 0x143;    // row_bcast:31

__device__ __forceinline__ float read_lane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<kDppQuadSwap1>(v, v));
  v = fmaxf(v, dpp_move<kDppQuadSwap2>(v, v));
  v = fmaxf(v, dpp_move<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_move<kDppRowMirror>(v, v));
  v = fmaxf(v, dpp_move<kDppBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp_move<kDppBcast31, 0xc>(v, v));
  return read_lane(v, 63);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<kDppQuadSwap1>(0.f, v);
  v += dpp_move<kDppQuadSwap2>(0.f, v);
  v += dpp_move<kDppHalfMirror>(0.f, v);
  v += dpp_move<kDppRowMirror>(0.f, v);
  v += dpp_move<kDppBcast15, 0xa>(0.f, v);
  v += dpp_move<kDppBcast31, 0xc>(0.f, v);
  return read_lane(v, 63);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the wave's lanes on DPP moves: the sums of up to
// four lanes (row shifts by 1, 2, 3), then row shifts by 4 and 8 on the upper
// banks, then the two row broadcasts.  Every lane must be active.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ int dpp_move_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  int s = v + dpp_move_i<0x111>(v);
  s += dpp_move_i<0x112>(v);
  s += dpp_move_i<0x113>(v);
  s += dpp_move_i<0x114, 0xf, 0xe>(s);
  s += dpp_move_i<0x118, 0xf, 0xc>(s);
  s += dpp_move_i<kDppBcast15, 0xa>(s);
  s += dpp_move_i<kDppBcast31, 0xc>(s);
  return s;
}
__device__ __forceinline__ int read_lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// The entry that ranks first among a wave's MPL values per lane (entry
// lane + 64*m; larger value first, lower entry number on equal values, -0 ==
// +0), skipping entries at or past n and those marked in `taken` (bit m).
// Returns the entry number (uniform) and its value in `best`.
template <int MPL>
__device__ __forceinline__ int wave_argmax(const float (&v)[MPL], int n, uint32_t taken, float &best) {
  const int lane = threadIdx.x & (kWave - 1);
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < MPL; ++m)
    if (lane + kWave * m < n && !((taken >> m) & 1u)) mx = fmaxf(mx, v[m]);
  mx = wave_max(mx);
  best = mx;
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const uint64_t hit = __ballot(lane + kWave * m < n && !((taken >> m) & 1u) && v[m] == mx);
    if (hit) return kWave * m + __builtin_ctzll(hit);
  }
  return -1;  // only when fewer than one untaken entry remains
}

// Sigmoid and SiLU on the hardware exp2 and reciprocal (a few ulp of fp32;
// the per-op bf16 rounding that follows in the rounded SwiGLU hides them).
__device__ __forceinline__ float sigmoid_f32(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504f));
}
__device__ __forceinline__ float silu_f32(float g) { return g * sigmoid_f32(g); }

// tanh-form GELU, 0.5 g (1 + tanh(z)) with z = sqrt(2/pi) (g + 0.044715 g^3),
// written as g * sigmoid(2z) (the identity 0.5 (1 + tanh z) = 1 / (1 + e^-2z)).
__device__ __forceinline__ float gelu_tanh_f32(float g) {
  const float z2 = 1.5957691216057308f * __builtin_fmaf(0.044715f * g, g * g, g);
  return g * sigmoid_f32(z2);
}

// Per-op rounding modes of the gated unit: none, or to the layer's 16-bit
// activation dtype.
constexpr int kRoundNone = 0, kRoundBF16 = 1, kRoundF16 = 2;
__device__ __forceinline__ float round_f16(float f) { return float(_Float16(f)); }
__device__ __forceinline__ float round_mode(float f, int mode) {
  return mode == kRoundF16 ? round_f16(f) : round_bf16(f);
}

// The gated unit of one (gate, up) pair: SwiGLU, silu(g) * u, or GeGLU,
// gelu_tanh(g) * u.  With per-op rounding (mode bf16 or fp16): gate and up
// rounded, then for SwiGLU sigmoid, g*s and (g*s)*u each rounded; for GeGLU
// gelu(g) and gelu(g)*u each rounded (round to nearest even).
template <int MODE, bool GEGLU>
__device__ __forceinline__ float glu_t(float g, float u) {
  if constexpr (MODE == kRoundNone) {
    return (GEGLU ? gelu_tanh_f32(g) : silu_f32(g)) * u;
  } else {
    auto r = [](float v) { return MODE == kRoundF16 ? round_f16(v) : round_bf16(v); };
    g = r(g);
    u = r(u);
    if constexpr (GEGLU) return r(r(gelu_tanh_f32(g)) * u);
    const float s = r(sigmoid_f32(g));
    const float a = r(g * s);
    return r(a * u);
  }
}
__device__ __forceinline__ float glu(float g, float u, int round_mode_, bool geglu) {
  if (round_mode_ == kRoundNone) return geglu ? glu_t<kRoundNone, true>(g, u) : glu_t<kRoundNone, false>(g, u);
  if (round_mode_ == kRoundF16) return geglu ? glu_t<kRoundF16, true>(g, u) : glu_t<kRoundF16, false>(g, u);
  return geglu ? glu_t<kRoundBF16, true>(g, u) : glu_t<kRoundBF16, false>(g, u);
}

// Calls f(std::integral_constant<int, mode>, std::integral_constant<bool, geglu>)
// for the run-time rounding mode and gate function, so that a loop over many
// outputs is compiled once per case instead of selecting per value.
template <typename F>
__device__ __forceinline__ void with_glu(int round_mode_, bool geglu, F &&f) {
  using N = std::integral_constant<int, kRoundNone>;
  using B = std::integral_constant<int, kRoundBF16>;
  using H = std::integral_constant<int, kRoundF16>;
  using T = std::true_type;
  using Fl = std::false_type;
  if (round_mode_ == kRoundBF16) {
    if (geglu) f(B{}, T{}); else f(B{}, Fl{});
  } else if (round_mode_ == kRoundF16) {
    if (geglu) f(H{}, T{}); else f(H{}, Fl{});
  } else {
    if (geglu) f(N{}, T{}); else f(N{}, Fl{});
  }
}


// The gate's activation a(g) and its derivative a'(g), fp32 with the
// library's expf / tanhf: SiLU, a = g s with s = sigmoid(g), a' = s (1 + g (1 - s));
// tanh-GELU, a = g (1 + th) / 2 with th = tanh(z), z = c (g + 0.044715 g^3),
// a' = (1 + th) / 2 + g (1 - th^2) c (1 + 3 * 0.044715 g^2) / 2, c = sqrt(2/pi).
__device__ __forceinline__ void gate_act_grad(float g, bool geglu, float &act, float &dact) {
  if (geglu) {
    const float ca = 0.7978845608028654f, cb = 0.044715f;
    const float th = tanhf(ca * __builtin_fmaf(cb * g, g * g, g));
    act = 0.5f * g * (1.0f + th);
    dact = 0.5f * (1.0f + th) + 0.5f * g * (1.0f - th * th) * ca * __builtin_fmaf(3.0f * cb, g * g, 1.0f);
  } else {
    const float s = 1.0f / (1.0f + expf(-g));
    act = g * s;
    dact = s * __builtin_fmaf(g, 1.0f - s, 1.0f);
  }
}

}  // namespace moe
