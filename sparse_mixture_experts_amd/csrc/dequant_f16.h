// dequant_f16.h -- affine code expansion to fp16 for the matrix-core kernels.
//
// A pair of codes is placed under the fp16 exponent of 1024 (the code in the
// low mantissa bits), 1024 is subtracted exactly and one packed fma gives
// s*q + b for both codes.  Eight codes come out in the order
// q0,q4,q1,q5,q2,q6,q3,q7, so activations are staged with the same order
// inside every 8-element block (permute8 in f16_stage.h).
#pragma once

#include "device_common.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 codes of a word -> 8 fp16 weights s*q + b in the order q0,q4,q1,q5,q2,q6,q3,q7.
// Codes 0/4 and 2/6 (after a shift by 8) sit in mantissa bits 0-3 of the two
// halves: OR-ing the fp16 exponent of 1024 gives 1024 + q.  Codes 1/5 and
// 3/7 sit in bits 4-7: the same OR gives 1024 + 16q, used with s/16.  Both
// subtractions of 1024 are exact, and each fma rounds s*q + b once.  `magic`
// holds 0x64006400 in a register so that every mask-and-or is one
// v_and_or_b32 with a single literal.
__device__ __forceinline__ f16x8 q4_word_to_f16(uint32_t w, h2 s2, h2 s2_16, h2 b2, uint32_t magic) {
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t w8 = w >> 8;
  const uint32_t c[4] = {(w & 0x000f000fu) | magic, (w & 0x00f000f0u) | magic, (w8 & 0x000f000fu) | magic,
                         (w8 & 0x00f000f0u) | magic};
  h2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_elementwise_fma(__builtin_bit_cast(h2, c[j]) - k1024, (j & 1) ? s2_16 : s2, b2);
  return __builtin_bit_cast(f16x8, r);
}

// 8 codes of two words (columns 0-3 in w0, 4-7 in w1) -> 8 fp16 weights s*q + b
// in the same order q0,q4,q1,q5,q2,q6,q3,q7 as q4_word_to_f16.  One byte
// permute interleaves the two words' low (high) halves, and one more per pair
// places two codes under the fp16 exponent bytes of 1024 (held in `mg` as
// 0x64646464): 1024 + q exactly, for q <= 255.
__device__ __forceinline__ f16x8 q8_words_to_f16(uint32_t w0, uint32_t w1, h2 s2, h2 b2, uint32_t mg) {
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  // __builtin_amdgcn_perm(hi, lo, sel): selector byte i picks byte sel_i of
  // the 8-byte value hi:lo (0-3 from lo, 4-7 from hi) for result byte i.
  const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // q0, q4, q1, q5
  const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // q2, q6, q3, q7
  const uint32_t c[4] = {__builtin_amdgcn_perm(mg, t0, 0x04010400u), __builtin_amdgcn_perm(mg, t0, 0x04030402u),
                         __builtin_amdgcn_perm(mg, t1, 0x04010400u), __builtin_amdgcn_perm(mg, t1, 0x04030402u)};
  h2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_elementwise_fma(__builtin_bit_cast(h2, c[j]) - k1024, s2, b2);
  return __builtin_bit_cast(f16x8, r);
}

// The expansions of the tile-packed fast path: 8 fp16 values
// round(s*(q - z) + delta), z = 8 (4-bit) or 128 (8-bit), each from one fma
// on 1024 + q with the addend n2 = round(-(1024 + z) s) (one pk_mul of s by
// the exact constant); the fma forms s*(1024 + q) + n2 = s*(q - z) + delta
// exactly (delta = n2 + (1024 + z) s, |delta| <= |s|) and rounds once.  The
// rest of each weight, b - 1024 s - n2, is the same for the whole group and
// enters as a separate product with the group sums of the activations.
// Order q0,q4,q1,q5,q2,q6,q3,q7 as above; every 4-bit code is shifted to the
// low nibble of its half (three shifts), so that all use the same n2.
__device__ __forceinline__ f16x8 q4_word_to_f16_c(uint32_t w, h2 s2, h2 n2, uint32_t magic) {
  const uint32_t c[4] = {(w & 0x000f000fu) | magic, ((w >> 4) & 0x000f000fu) | magic,
                         ((w >> 8) & 0x000f000fu) | magic, ((w >> 12) & 0x000f000fu) | magic};
  h2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_elementwise_fma(__builtin_bit_cast(h2, c[j]), s2, n2);
  return __builtin_bit_cast(f16x8, r);
}
__device__ __forceinline__ f16x8 q8_words_to_f16_c(uint32_t w0, uint32_t w1, h2 s2, h2 n2, uint32_t mg) {
  const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // q0, q4, q1, q5
  const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // q2, q6, q3, q7
  const uint32_t c[4] = {__builtin_amdgcn_perm(mg, t0, 0x04010400u), __builtin_amdgcn_perm(mg, t0, 0x04030402u),
                         __builtin_amdgcn_perm(mg, t1, 0x04010400u), __builtin_amdgcn_perm(mg, t1, 0x04030402u)};
  h2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_elementwise_fma(__builtin_bit_cast(h2, c[j]), s2, n2);
  return __builtin_bit_cast(f16x8, r);
}

}  // namespace moe
