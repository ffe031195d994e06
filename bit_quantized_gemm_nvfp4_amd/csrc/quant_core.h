// quant_core.h -- the NVFP4 activation-quantizer rule as device functions
// (internal), shared by the quantize kernels and the GEMV's fused W4A4
// activation staging.
//
// Per block of 16 elements ("52.6% more tokens, 1.53x less GPU time:
// production inference with Minima and Rafay": NVFP4 W4A4 execution; format:
// "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding head",
// section "What the artifact is"): scale = the block's max |x| / 6 rounded to
// the nearest E4M3 value (ties to the even code, saturating at 448), codes =
// the e2m1 magnitude nearest to |x| / scale (ties to the even index,
// saturating at 6) with the sign of x.
#pragma once

#include "device.h"

namespace nvfp4 {

// Scale code for a block maximum a (finite, >= 0): a/6 rounded to the nearest
// E4M3 value, ties to the even code, saturating at 448 (0x7E).
//   t = a / 6 is a correctly rounded f32 division.  It cannot move the value
//   across an E4M3 rounding boundary: a boundary t* has at most 5 significant
//   bits, so a = 6 t* is exact and then t == t*; any other bf16 a lies at least
//   a relative 2^-8 away from 6 t*, far beyond the 2^-24 division error.
//   Subnormal range (t < 2^-6): the code is the integer nearest t / 2^-9
//   (0..8; 8 is 2^-6 = code 0x08).  Normal range: round the f32 mantissa to 3
//   bits, nearest-even, on the bit pattern, and rebias the exponent 127 -> 7.
//   A NaN maximum (the block holds a NaN) gives the NaN code 0x7F, so the
//   block decodes to NaN and the code never spills past its 8 bits.
__device__ __forceinline__ uint32_t scale_code_from_amax(float a) {
  float t = a / 6.0f;
  if (t != t) return 0x7F;
  if (t >= 448.0f) return 0x7E;
  if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);
  uint32_t b = __builtin_bit_cast(uint32_t, t);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  return r - (120u << 3);
}

// Magnitude index (0..7) of the e2m1 value nearest to ax / s, ties to the even
// index, saturating at 6.  The decision points are s * {0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5}; each product is exact in f32, so every comparison is
// exact.  A tie at 0.75, 1.75, 3.5 resolves upward (to the even index 2, 4, 6)
// and at 0.25, 1.25, 2.5, 5 downward (to 0, 2, 4, 6), hence >= vs >.
// Three comparisons pick the index bit by bit.
struct Thresholds {
  float t025, t075, t125, t175, t250, t350, t500;
};

__device__ __forceinline__ Thresholds make_thresholds(float s) {
  return {s * 0.25f, s * 0.75f, s * 1.25f, s * 1.75f, s * 2.5f, s * 3.5f, s * 5.0f};
}

__device__ __forceinline__ uint32_t e2m1_index(float ax, const Thresholds& th) {
  bool hi = ax >= th.t175;                          // index >= 4
  bool mid = ax >= (hi ? th.t350 : th.t075);         // next bit
  float t3 = hi ? (mid ? th.t500 : th.t250) : (mid ? th.t125 : th.t025);
  bool lo = ax > t3;
  return (hi ? 4u : 0u) | (mid ? 2u : 0u) | (lo ? 1u : 0u);
}

// The 8 codes of one 16-byte piece (8 bf16 values) under its block's scale
// code sc (value s): element e in nibble e, so element 2j is the low nibble
// of byte j.
__device__ __forceinline__ uint32_t piece_codes(u32x4 v, uint32_t sc, float s) {
  const Thresholds th = make_thresholds(s);
  uint32_t codes = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t bits = (v[i] >> (16 * h)) & 0xFFFFu;
      const uint32_t mag = (sc == 0) ? 0u : e2m1_index(bf16_bits_to_f32(bits & 0x7FFFu), th);
      codes |= (mag | ((bits >> 12) & 8u)) << (4 * (2 * i + h));
    }
  }
  return codes;
}

// The 8 values of one 16-byte piece quantized with a block's scale code sc
// and dequantized: e2m1(code) * e4m3(sc) rounded to bf16 (exact).
__device__ __forceinline__ u32x4 fakequant_with(u32x4 v, uint32_t sc) {
  const float s = e4m3_to_f32<0>(sc);
  return dequant8_bf16(piece_codes(v, sc, s), s);
}

__device__ __forceinline__ uint32_t piece_amax_bits(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
  return m;  // non-negative finite bf16: integer order
}

// Scale code of the block whose two 16-byte pieces sit in this lane and the
// neighbouring one (lane ^ 1): both lanes must be active.
__device__ __forceinline__ uint32_t pair_scale_code(u32x4 v) {
  uint32_t amax_bits = piece_amax_bits(v);
  amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 1, 64));
  return scale_code_from_amax(bf16_bits_to_f32(amax_bits));
}

// Fake quantization of one 16-byte piece (8 bf16 values) of a block whose
// other 8 values sit in the neighbouring lane (lane ^ 1): both lanes must be
// active.  Returns the 8 values quantized and dequantized, bit-identical to
// nvfp4_quantize followed by nvfp4_dequantize.
__device__ __forceinline__ u32x4 fakequant_piece(u32x4 v) {
  return fakequant_with(v, pair_scale_code(v));
}

// The same for a whole block held by one thread (pieces v0, v1).
__device__ __forceinline__ void fakequant_block(u32x4& v0, u32x4& v1) {
  const uint32_t sc =
      scale_code_from_amax(bf16_bits_to_f32(max(piece_amax_bits(v0), piece_amax_bits(v1))));
  v0 = fakequant_with(v0, sc);
  v1 = fakequant_with(v1, sc);
}

}  // namespace nvfp4
