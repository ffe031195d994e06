// device.h -- gfx950 device helpers shared by the NVFP4 kernels (internal).
//
// NVFP4: 4-bit e2m1 elements, one FP8 E4M3 scale per 16 consecutive
// K-elements ("Serving Qwen3.8-27B in 4-bit with a masked speculative
// decoding head", section "What the artifact is"; E4M3 = 4 exponent and 3
// mantissa bits: "What 350+ Experiments Taught Us About Serving Qwen 3.6
// 35B-A3B", section 3).
//
// Decoding on gfx950:
//  * v_cvt_f32_fp8 decodes an OCP E4M3FN byte to f32 exactly (all 256 codes,
//    NaN for 0x7F/0xFF).
//  * v_cvt_scalef32_pk_{f32,bf16}_fp4 decode two e2m1 nibbles of one byte
//    (low nibble -> element 0) exactly, but apply only the EXPONENT of their
//    f32 scale operand (the scale behaves like an E8M0 power of two).  An
//    E4M3 scale has a 3-bit mantissa, so the per-16 scale is applied with an
//    ordinary f32 multiply (or on the accumulator), never through that operand.
//  * e2m1 * e4m3 has <= 6 significant bits within [2^-10, 2688]: exact in f32
//    and in bf16, so dequantized operands are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// E4M3 byte `sel` (0..3) of `w` -> f32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// Two e2m1 codes in byte SEL of w -> f32 pair (exact, unscaled).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Two e2m1 codes in byte SEL of w -> bf16 pair (exact, unscaled).
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight consecutive elements (one 32-bit word of codes) times one f32 scale
// -> eight exact bf16 values, element order preserved (word i holds elements
// 2i, 2i+1 in its low/high half).
__device__ __forceinline__ u32x4 dequant8_bf16(uint32_t codes, float s) {
  f32x2 p0 = e2m1x2_to_f32<0>(codes);
  f32x2 p1 = e2m1x2_to_f32<1>(codes);
  f32x2 p2 = e2m1x2_to_f32<2>(codes);
  f32x2 p3 = e2m1x2_to_f32<3>(codes);
  u32x4 r;
  r[0] = pack_bf16x2(p0[0] * s, p0[1] * s);
  r[1] = pack_bf16x2(p1[0] * s, p1[1] * s);
  r[2] = pack_bf16x2(p2[0] * s, p2[1] * s);
  r[3] = pack_bf16x2(p3[0] * s, p3[1] * s);
  return r;
}

// The same eight elements in fp16: e2m1 codes decoded exactly to fp16, then one
// packed fp16 multiply per pair by the E4M3 scale s (exact in fp16: the
// product has <= 6 significant bits within [2^-10, 2688], inside fp16's normal
// range).  Half the vector instructions of dequant8_bf16.
__device__ __forceinline__ u32x4 dequant8_f16(uint32_t codes, _Float16 s) {
  const f16x2 ss = {s, s};
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss);
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss);
  return r;
}

// E4M3 bytes 0,1 (HI = false) or 2,3 (HI = true) of w -> fp16 pair (exact).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight bf16 values -> fp16.  Returns true when every value is represented
// exactly (then an fp16 product equals the bf16 one); false for values out of
// fp16's range, below its precision, or non-finite.
__device__ __forceinline__ bool bf16x8_to_f16(const u32x4& v, u32x4& h) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, v[i] << 16);
    const float hi = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
    const f16x2 p = {(_Float16)lo, (_Float16)hi};
    ok = ok && ((float)p.x == lo) && ((float)p.y == hi);
    h[i] = __builtin_bit_cast(uint32_t, p);
  }
  return ok;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __builtin_bit_cast(float, h16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Output multiplier of a product of two-level NVFP4 tensors: *a * *w (a null
// pointer stands for 1).  Callers multiply only when either pointer is set.
__device__ __forceinline__ float alpha_of(const float* a, const float* w) {
  return (a ? *a : 1.0f) * (w ? *w : 1.0f);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup barrier that publishes LDS data.  The wave first waits until at
// most kVm of its vector-memory operations are outstanding (kVm >= 0; its
// global->LDS copies must be older than those kVm), then for its own LDS
// accesses (LDS-only release fence), then meets the other waves.  Unlike
// __syncthreads() it leaves the other global loads in flight.
template <int kVm>
__device__ __forceinline__ void lds_barrier() {
  static_assert(kVm < 64, "vmcnt has 6 bits");
  if constexpr (kVm >= 0)  // s_waitcnt vmcnt(kVm) expcnt(7) lgkmcnt(15)
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | 0x0F70);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace nvfp4
