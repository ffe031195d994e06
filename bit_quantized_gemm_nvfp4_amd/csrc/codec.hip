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
#include "quant_core.h"

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

// Launches that fit one round of the chip (kPiecesMax lanes, 8 resident
// 256-thread workgroups per CU) are bound by each thread's serial instruction
// stream, not by memory: they take one lane per 8 elements (one 16-byte piece
// of bf16) instead of 32 or 16 per thread.  Larger ones keep the wider
// threads, which move the same bytes with fewer instructions.
constexpr int64_t kPiecesMax = 256 * 8 * 256;

// One lane per 8 elements: 4 code bytes and the block's scale byte in, one
// 16-byte piece of bf16 out.
__global__ void __launch_bounds__(256) k_dequantize_pieces(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t pieces,
                                                           uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= pieces) return;
  const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[t];
  const float s = e4m3_to_f32<0>((uint32_t)scales[t >> 1]);
  reinterpret_cast<u32x4*>(out)[t] = dequant8_bf16(w, s);
}

int launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                      uint16_t* out, hipStream_t stream) {
  const int64_t pieces = N * (K / 8);
  if (pieces <= kPiecesMax) {
    hipLaunchKernelGGL(k_dequantize_pieces, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       stream, codes, scales, pieces, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  int64_t cpr = K / 32, total = N * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales,
                     cpr, total, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- quantize ---------------------------------------------------------------------

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

// One lane per 8 elements: the two lanes of a 16-element block exchange their
// maxima, each writes its 4 code bytes and the even one the scale byte.  The
// element count is a multiple of 32 (K % 32 == 0), so the lanes of a block
// are present or absent together.
__global__ void __launch_bounds__(256) k_quantize_pieces(const uint16_t* __restrict__ x,
                                                         int64_t pieces,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= pieces) return;
  const u32x4 v = reinterpret_cast<const u32x4*>(x)[t];
  const uint32_t sc = pair_scale_code(v);
  reinterpret_cast<uint32_t*>(codes)[t] = piece_codes(v, sc, e4m3_to_f32<0>(sc));
  if ((t & 1) == 0) scales[t >> 1] = (uint8_t)sc;
}

int launch_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                    hipStream_t stream) {
  const int64_t pieces = M * (K / 8);
  if (pieces <= kPiecesMax) {
    hipLaunchKernelGGL(k_quantize_pieces, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       stream, x, pieces, codes, scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  int64_t cpr = K / 32, total = M * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, x, cpr, total,
                     codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- fake quantization: x -> dequantize(quantize(x)) in bf16, one pass ---------------

// One thread per 16-element block: two 16-byte loads, two 16-byte stores.
__global__ void __launch_bounds__(256) k_fakequant(const uint16_t* __restrict__ x,
                                                   int64_t blocks, uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= blocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + t * 16);
  u32x4 v0 = src[0], v1 = src[1];
  fakequant_block(v0, v1);
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * 16);
  dst[0] = v0;
  dst[1] = v1;
}

// One lane per 8 elements (fakequant_piece: the block's two lanes exchange
// their maxima).
__global__ void __launch_bounds__(256) k_fakequant_pieces(const uint16_t* __restrict__ x,
                                                          int64_t pieces,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= pieces) return;
  reinterpret_cast<u32x4*>(out)[t] = fakequant_piece(reinterpret_cast<const u32x4*>(x)[t]);
}

int launch_fakequant(const uint16_t* x, int64_t M, int64_t K, uint16_t* out, hipStream_t stream) {
  const int64_t pieces = M * (K / 8);
  if (pieces <= kPiecesMax) {
    hipLaunchKernelGGL(k_fakequant_pieces, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       stream, x, pieces, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int64_t blocks = M * (K / 16);
  hipLaunchKernelGGL(k_fakequant, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream, x,
                     blocks, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- two-level NVFP4: a per-tensor fp32 scale g above the per-16 scales ------------
//
// An element is e2m1(code) * e4m3(scale) * g.  Quantizing with g divides
// every element by g in binary32 (correctly rounded), y = fl32(x / g), and
// applies the single-level rule above to y.  scale_code_from_amax stays exact
// for binary32 inputs: a binary32 a other than 6 t* lies at least ulp(a) away
// from it, more than twice the error of fl32(a / 6).  The offline weight
// quantizer takes g = fl32(amax / 2688) (2688 = 6 * 448), or 1 for an
// all-zero tensor.

// 16 binary32 values -> scale code and 8 code bytes (2 words).
__device__ __forceinline__ uint32_t quantize_block_f32(const float (&y)[16], u32x2& codes_out) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)  // non-negative finite binary32: integer order
    amax_bits = max(amax_bits, __float_as_uint(y[i]) & 0x7FFFFFFFu);
  const uint32_t sc = scale_code_from_amax(__uint_as_float(amax_bits));
  const Thresholds th = make_thresholds(e4m3_to_f32<0>(sc));
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bits = __float_as_uint(y[e]);
    const uint32_t mag = (sc == 0) ? 0u : e2m1_index(__uint_as_float(bits & 0x7FFFFFFFu), th);
    packed[e >> 3] |= (mag | ((bits >> 28) & 8u)) << (4 * (e & 7));
  }
  codes_out[0] = packed[0];
  codes_out[1] = packed[1];
  return sc;
}

__global__ void __launch_bounds__(256) k_quantize_scaled(const uint16_t* __restrict__ x,
                                                         int64_t chunks_per_row,
                                                         int64_t total_chunks,
                                                         const float* __restrict__ g,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_chunks) return;
  const float gv = *g;
  int64_t m = t / chunks_per_row;
  int64_t c = t - m * chunks_per_row;
  const int64_t K = chunks_per_row * 32;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + m * K + c * 32);
  uint32_t sc[2];
  u32x2 cw[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const u32x4 v0 = src[2 * b], v1 = src[2 * b + 1];
    const uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    float y[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu) / gv;
      y[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16) / gv;
    }
    sc[b] = quantize_block_f32(y, cw[b]);
  }
  *reinterpret_cast<u32x4*>(codes + m * (K / 2) + c * 16) = u32x4{cw[0][0], cw[0][1], cw[1][0],
                                                                  cw[1][1]};
  *reinterpret_cast<uint16_t*>(scales + m * (K / 16) + c * 2) = (uint16_t)(sc[0] | (sc[1] << 8));
}

// Largest |x| (as bf16 magnitude bits) over a grid-stride part of n8 words of
// 8 bf16 values; one partial per workgroup.
__global__ void __launch_bounds__(256) k_absmax_partial(const uint16_t* __restrict__ x, int64_t n8,
                                                        uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[256];
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// g = fl32(amax / 2688) from the partials, or 1 for an all-zero tensor.
__global__ void __launch_bounds__(256) k_global_scale(const uint32_t* __restrict__ partial,
                                                      int parts, float* __restrict__ g) {
  __shared__ uint32_t red[256];
  uint32_t mx = 0;
  for (int i = threadIdx.x; i < parts; i += blockDim.x) mx = max(mx, partial[i]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float a = bf16_bits_to_f32(red[0]);
    *g = a > 0.0f ? a / 2688.0f : 1.0f;
  }
}

// out = bf16(fl32(e2m1 * e4m3 * g)): the first product is exact, the second
// rounds once.
__global__ void __launch_bounds__(256) k_dequantize_scaled(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ g,
                                                           int64_t chunks_per_row,
                                                           int64_t total_chunks,
                                                           uint16_t* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_chunks) return;
  const float gv = *g;
  int64_t n = t / chunks_per_row;
  int64_t c = t - n * chunks_per_row;
  const int64_t K = chunks_per_row * 32;
  const u32x4 w = *reinterpret_cast<const u32x4*>(codes + n * (K / 2) + c * 16);
  const uint32_t sc = *reinterpret_cast<const uint16_t*>(scales + n * (K / 16) + c * 2);
  const float s[2] = {e4m3_to_f32<0>(sc), e4m3_to_f32<1>(sc)};
  u32x4* o = reinterpret_cast<u32x4*>(out + n * K + c * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sq = s[q >> 1];
    const f32x2 p0 = e2m1x2_to_f32<0>(w[q]), p1 = e2m1x2_to_f32<1>(w[q]);
    const f32x2 p2 = e2m1x2_to_f32<2>(w[q]), p3 = e2m1x2_to_f32<3>(w[q]);
    o[q] = u32x4{pack_bf16x2((p0[0] * sq) * gv, (p0[1] * sq) * gv),
                 pack_bf16x2((p1[0] * sq) * gv, (p1[1] * sq) * gv),
                 pack_bf16x2((p2[0] * sq) * gv, (p2[1] * sq) * gv),
                 pack_bf16x2((p3[0] * sq) * gv, (p3[1] * sq) * gv)};
  }
}

int launch_quantize_scaled(const uint16_t* x, int64_t M, int64_t K, const float* g,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  int64_t cpr = K / 32, total = M * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_quantize_scaled, dim3((unsigned)blocks), dim3(256), 0, stream, x, cpr,
                     total, g, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

size_t quantize_weight_workspace_bytes() { return kAbsmaxParts * sizeof(uint32_t); }

int launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* scales, float* g, void* workspace, hipStream_t stream) {
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const int64_t n8 = N * K / 8;
  int parts = (int)((n8 + 255) / 256);
  if (parts > kAbsmaxParts) parts = kAbsmaxParts;
  hipLaunchKernelGGL(k_absmax_partial, dim3((unsigned)parts), dim3(256), 0, stream, w, n8,
                     partial);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(k_global_scale, dim3(1), dim3(256), 0, stream, partial, parts, g);
  if (hipGetLastError() != hipSuccess) return -1;
  return launch_quantize_scaled(w, N, K, g, codes, scales, stream);
}

int launch_dequantize_scaled(const uint8_t* codes, const uint8_t* scales, const float* g,
                             int64_t N, int64_t K, uint16_t* out, hipStream_t stream) {
  int64_t cpr = K / 32, total = N * cpr;
  int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_dequantize_scaled, dim3((unsigned)blocks), dim3(256), 0, stream, codes,
                     scales, g, cpr, total, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
