// Device helpers for MXFP8 on gfx950: scale rule, BF16 -> E4M3 encoding, fp32 -> BF16 rounding.
//
// MXFP8 here is one OCP E4M3FN byte per element plus one UE8M0 scale byte per
// 32 contiguous elements of a row (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn:
// wo_a writes wo_b's MXFP8 input", Conversation; vLLM PR #57977
// "[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM kernels", Pieces).
// The scale exponent of a block is the smallest e with max|x| <= 448 * 2^e,
// clamped to [-127, 127]; the codes are x / 2^e rounded to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Scale exponent of a block from its largest magnitude, given as BF16 bits with
// the sign cleared (for non-negative floats the bit order is the value order).
// With amax = (1 + m/128) * 2^(E-127): amax <= 1.75 * 2^(e+8) gives
// e = E - 135 when m <= 0x60 (1 + m/128 <= 1.75) and E - 134 above that; the
// BF16 subnormals (E == 0) and everything below 448 * 2^-127 clamp to -127.
// BF16's largest finite value gives 120, so the upper clamp is never reached.
__device__ __forceinline__ int scale_exp_from_amax(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 7);
  int e = E - 135 + ((amax_bits & 0x7Fu) > 0x60u ? 1 : 0);
  e = e < -127 ? -127 : e;
  return E == 0 ? -127 : e;
}

// 2^e as an fp32 for e in [-127, 127]; 2^-127 is the subnormal 0x00400000.
__device__ __forceinline__ float exp2_int(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Largest magnitude (BF16 bits, sign cleared) of the two BF16 values packed in a word.
__device__ __forceinline__ uint32_t amax_pair(uint32_t acc, uint32_t pair) {
  const u16x2 a = __builtin_bit_cast(u16x2, acc);
  const u16x2 b = __builtin_bit_cast(u16x2, pair & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t fold_pair(uint32_t acc) {
  const uint32_t lo = acc & 0xFFFFu, hi = acc >> 16;
  return lo > hi ? lo : hi;
}

// Four BF16 values (two packed pairs, element 0 in the low half) -> four E4M3
// bytes (element 0 in the low byte): RNE of x / scale, saturating.  gfx950's
// scaled conversion divides by the fp32 scale exactly; it matches the
// reference rounding on every BF16 value at every scale 2^e, e in [-127, 127].
__device__ __forceinline__ uint32_t encode4(uint32_t p01, uint32_t p23, float scale) {
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((v2s){0, 0}, __builtin_bit_cast(v2bf, p01), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, p23), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Two fp32 values -> two BF16 values packed in a word (a in the low half), round to nearest even,
// with gfx950's packed conversion (v_cvt_pk_bf16_f32): one instruction instead of about seven for
// the integer formula (u + 0x7FFF + bit 16 of u) >> 16, which it matches on every finite fp32 bit
// pattern, subnormals and overflow to infinity included (checked on the device exhaustively).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

}  // namespace mx
