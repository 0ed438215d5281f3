// device_common.h -- small device helpers for the gfx950 kernels: bf16
// conversions and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }
// The two bf16 values packed in a 32-bit word (element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }

// Activation element i as fp32 (BF16: array of bf16 bits).
template <bool BF16>
__device__ __forceinline__ float load_act(const void *p, int64_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

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

// The gated unit of one (gate, up) pair: SwiGLU, silu(g) * u, or GeGLU,
// gelu_tanh(g) * u.  With per-op rounding: gate and up rounded to bf16, then
// for SwiGLU sigmoid, g*s and (g*s)*u each rounded to bf16; for GeGLU
// gelu(g) and gelu(g)*u each rounded to bf16.
__device__ __forceinline__ float glu(float g, float u, bool round_ops, bool geglu) {
  if (!round_ops) return (geglu ? gelu_tanh_f32(g) : silu_f32(g)) * u;
  g = round_bf16(g);
  u = round_bf16(u);
  if (geglu) return round_bf16(round_bf16(gelu_tanh_f32(g)) * u);
  float s = round_bf16(sigmoid_f32(g));
  float a = round_bf16(g * s);
  return round_bf16(a * u);
}

}  // namespace moe
