// codec.hip -- NVFP4 dequantize and quantize kernels for gfx950.
//
// Format: "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding
// head", section "What the artifact is" (e2m1 elements, one FP8 scale per 16);
// "What 350+ Experiments Taught Us About Serving Qwen 3.6 35B-A3B", section 3
// (E4M3).  Activation quantization is the W4A4 path of "52.6% more tokens,
// 1.53x less GPU time: production inference with Minima and Rafay".
//
// Both kernels move 32 consecutive elements of one row per thread (one
// 16-byte word of codes, two scale bytes, 64 bytes of bf16): consecutive
// threads touch consecutive memory, so every load and store is a coalesced
// 128-bit access.  Both are HBM-bound.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

// ---- dequantize: out[n][k] = e2m1(code) * e4m3(scale) --------------------------

__global__ void __launch_bounds__(256) k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    int64_t chunks_per_row, int64_t total_chunks,
                                                    uint16_t* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_chunks) return;
  int64_t n = t / chunks_per_row;
  int64_t c = t - n * chunks_per_row;
  const int64_t K = chunks_per_row * 32;
  u32x4 w = *reinterpret_cast<const u32x4*>(codes + n * (K / 2) + c * 16);
  uint32_t sc = *reinterpret_cast<const uint16_t*>(scales + n * (K / 16) + c * 2);
  float s0 = e4m3_to_f32<0>(sc);
  float s1 = e4m3_to_f32<1>(sc);
  u32x4* o = reinterpret_cast<u32x4*>(out + n * K + c * 32);
  o[0] = dequant8_bf16(w[0], s0);
  o[1] = dequant8_bf16(w[1], s0);
  o[2] = dequant8_bf16(w[2], s1);
  o[3] = dequant8_bf16(w[3], s1);
}

int launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                      uint16_t* out, hipStream_t stream) {
  int64_t cpr = K / 32, total = N * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales,
                     cpr, total, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- quantize ---------------------------------------------------------------------

// Scale code for a block maximum a (finite, >= 0): a/6 rounded to the nearest
// E4M3 value, ties to the even code, saturating at 448 (0x7E).
//   t = a / 6 is a correctly rounded f32 division.  It cannot move the value
//   across an E4M3 rounding boundary: a boundary t* has at most 5 significant
//   bits, so a = 6 t* is exact and then t == t*; any other bf16 a lies at least
//   a relative 2^-8 away from 6 t*, far beyond the 2^-24 division error.
//   Subnormal range (t < 2^-6): the code is the integer nearest t / 2^-9
//   (0..8; 8 is 2^-6 = code 0x08).  Normal range: round the f32 mantissa to 3
//   bits, nearest-even, on the bit pattern, and rebias the exponent 127 -> 7.
__device__ __forceinline__ uint32_t scale_code_from_amax(float a) {
  float t = a / 6.0f;
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

// 16 bf16 values (8 words) -> scale code and 8 code bytes (2 words).
__device__ __forceinline__ uint32_t quantize_block(const uint32_t (&xw)[8], u32x2& codes_out) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = xw[i] & 0x7FFFu, hi = (xw[i] >> 16) & 0x7FFFu;
    amax_bits = max(amax_bits, max(lo, hi));  // non-negative finite bf16: integer order
  }
  uint32_t sc = scale_code_from_amax(bf16_bits_to_f32(amax_bits));
  float s = e4m3_to_f32<0>(sc);
  Thresholds th = make_thresholds(s);
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t bits = (xw[i] >> (16 * h)) & 0xFFFFu;
      float ax = bf16_bits_to_f32(bits & 0x7FFFu);
      uint32_t mag = (sc == 0) ? 0u : e2m1_index(ax, th);
      uint32_t code = mag | ((bits >> 12) & 8u);
      int e = 2 * i + h;  // element index within the block
      packed[e >> 3] |= code << (4 * (e & 7));
    }
  }
  codes_out[0] = packed[0];
  codes_out[1] = packed[1];
  return sc;
}

__global__ void __launch_bounds__(256) k_quantize(const uint16_t* __restrict__ x,
                                                  int64_t chunks_per_row, int64_t total_chunks,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_chunks) return;
  int64_t m = t / chunks_per_row;
  int64_t c = t - m * chunks_per_row;
  const int64_t K = chunks_per_row * 32;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + m * K + c * 32);
  u32x4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
  uint32_t b0[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t b1[8] = {v2[0], v2[1], v2[2], v2[3], v3[0], v3[1], v3[2], v3[3]};
  u32x2 c0, c1;
  uint32_t s0 = quantize_block(b0, c0);
  uint32_t s1 = quantize_block(b1, c1);
  u32x4 cw = {c0[0], c0[1], c1[0], c1[1]};
  *reinterpret_cast<u32x4*>(codes + m * (K / 2) + c * 16) = cw;
  *reinterpret_cast<uint16_t*>(scales + m * (K / 16) + c * 2) = (uint16_t)(s0 | (s1 << 8));
}

int launch_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                    hipStream_t stream) {
  int64_t cpr = K / 32, total = M * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, x, cpr, total,
                     codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
