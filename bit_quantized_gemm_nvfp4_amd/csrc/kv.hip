// kv.hip -- FP8 E4M3 KV-cache codec for gfx950.
//
// The serving stacks keep the attention key/value cache as FP8 E4M3 in
// 16-token pages ("What 350+ Experiments Taught Us About Serving Qwen 3.6
// 35B-A3B", section 3 "KV cache and memory capacity"; E4M3 = 4 exponent and 3
// mantissa bits).  Two HBM-bound kernels:
//   store: bf16 token rows -> E4M3 codes at their cache slots,
//          code = E4M3(fl32(x / scale)), nearest, ties to even, satfinite;
//   load:  a batch of sequences gathered page by page through their block
//          tables -> bf16, value = bf16(fl32(e4m3 * scale)).
// A slot is page * page_size + position in the page, so the paged cache
// [pages][page_size][W] is addressed as rows [slot][W].  Each thread moves 16
// elements of one row: one 16-byte word of codes and two of bf16, so loads and
// stores are coalesced 128-bit accesses.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

namespace {

// E4M3 code of a binary32 value: nearest, ties to the even code, magnitudes
// at or above 448 saturate to 448 (0x7E), the sign is kept (zero included);
// a NaN gives the NaN code of its sign (0x7F / 0xFF).
//   Below 2^-6 (subnormal E4M3, spacing 2^-9): the magnitude is the integer
//   nearest |q| * 512 (exact scaling), 0..8, and 8 is the code of 2^-6.
//   Normal range: round the binary32 mantissa to 3 bits, nearest even, on
//   the bit pattern (a carry moves into the exponent), and rebias the
//   exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t a = b & 0x7FFFFFFFu;
  const float af = __uint_as_float(a);
  uint32_t c;
  if (af != af)
    c = 0x7Fu;
  else if (af >= 448.0f)
    c = 0x7Eu;
  else if (af < 0.015625f)
    c = (uint32_t)__builtin_rintf(af * 512.0f);
  else
    c = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  return ((b >> 24) & 0x80u) | c;
}

// q = v / d, r = v - q*d for 0 <= v < bound, d > 0 (d uniform).  When the
// index range and d fit 31 bits (a uniform test) the division is 32-bit, a
// few instructions instead of the long 64-bit sequence.
__device__ __forceinline__ void divmod_index(int64_t v, int64_t d, int64_t bound, int64_t& q,
                                             int64_t& r) {
  if (bound < ((int64_t)1 << 31) && d < ((int64_t)1 << 31)) {
    const uint32_t q32 = (uint32_t)v / (uint32_t)d;
    q = q32;
    r = (int64_t)((uint32_t)v - q32 * (uint32_t)d);
  } else {
    q = v / d;
    r = v - q * d;
  }
}

// 8 bf16 values (one 16-byte word) -> 8 codes (two 32-bit words).
__device__ __forceinline__ u32x2 encode8(u32x4 xw, float scale) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = bf16_bits_to_f32((xw[i] >> (16 * h)) & 0xFFFFu);
      const int e = 2 * i + h;
      w[e >> 2] |= e4m3_code(x / scale) << (8 * (e & 3));
    }
  }
  return u32x2{w[0], w[1]};
}

// 4 codes (one 32-bit word) -> 4 bf16 values (two 32-bit words).
__device__ __forceinline__ u32x2 decode4(uint32_t c, float scale) {
  return u32x2{pack_bf16x2(e4m3_to_f32<0>(c) * scale, e4m3_to_f32<1>(c) * scale),
               pack_bf16x2(e4m3_to_f32<2>(c) * scale, e4m3_to_f32<3>(c) * scale)};
}

__global__ void __launch_bounds__(256) k_kv_store(const uint16_t* __restrict__ x,
                                                  const int32_t* __restrict__ slot_mapping,
                                                  int64_t T, int64_t W, float scale,
                                                  uint8_t* __restrict__ cache, int64_t num_slots) {
  const int64_t per_row = W / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row, c = idx - t * per_row;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + t * W + c * 16);
  const u32x4 x0 = src[0], x1 = src[1];
  const u32x2 lo = encode8(x0, scale), hi = encode8(x1, scale);
  *reinterpret_cast<u32x4*>(cache + slot * W + c * 16) = u32x4{lo[0], lo[1], hi[0], hi[1]};
}

__global__ void __launch_bounds__(256) k_kv_load(const uint8_t* __restrict__ cache,
                                                 int64_t num_slots, int64_t W,
                                                 const int32_t* __restrict__ block_table,
                                                 const int32_t* __restrict__ seq_lens, int64_t B,
                                                 int64_t max_pages, int64_t page_size,
                                                 int64_t max_len, float scale,
                                                 uint16_t* __restrict__ out) {
  const int64_t per_row = W / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = B * max_len * per_row;
  if (idx >= n) return;
  int64_t row, c, b, i, page, pos;
  divmod_index(idx, per_row, n, row, c);
  divmod_index(row, max_len, n, b, i);
  divmod_index(i, page_size, n, page, pos);
  // the length and the page entry are loaded together (the entry is in the
  // table whenever its index is; it is used only below the length)
  const int32_t len = seq_lens[b];
  const int32_t entry = page < max_pages ? block_table[b * max_pages + page] : -1;
  int64_t slot = -1;
  if (i < len && entry >= 0) slot = (int64_t)entry * page_size + pos;
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * W + c * 16);
  if (slot < 0 || slot >= num_slots) {
    dst[0] = u32x4{0u, 0u, 0u, 0u};
    dst[1] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const u32x4 q = *reinterpret_cast<const u32x4*>(cache + slot * W + c * 16);
  const u32x2 d0 = decode4(q[0], scale), d1 = decode4(q[1], scale);
  const u32x2 d2 = decode4(q[2], scale), d3 = decode4(q[3], scale);
  dst[0] = u32x4{d0[0], d0[1], d1[0], d1[1]};
  dst[1] = u32x4{d2[0], d2[1], d3[0], d3[1]};
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

int launch_kv_store(const uint16_t* x, int64_t T, int64_t W, const int32_t* slot_mapping,
                    float scale, uint8_t* cache, int64_t num_slots, hipStream_t stream) {
  const int64_t threads = T * (W / 16);
  if (threads / 256 >= (int64_t)1 << 31) return -1;
  hipLaunchKernelGGL(k_kv_store, dim3(blocks_for(threads)), dim3(256), 0, stream, x,
                     slot_mapping, T, W, scale, cache, num_slots);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_kv_load(const uint8_t* cache, int64_t num_slots, int64_t W, const int32_t* block_table,
                   const int32_t* seq_lens, int64_t B, int64_t max_pages, int64_t page_size,
                   int64_t max_len, float scale, uint16_t* out, hipStream_t stream) {
  const int64_t threads = B * max_len * (W / 16);
  if (threads / 256 >= (int64_t)1 << 31) return -1;
  hipLaunchKernelGGL(k_kv_load, dim3(blocks_for(threads)), dim3(256), 0, stream, cache, num_slots,
                     W, block_table, seq_lens, B, max_pages, page_size, max_len, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
