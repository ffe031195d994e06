// gemv_core.h -- the weight-streaming inner loop shared by the decode GEMV and
// the grouped (mixture-of-experts) GEMV kernels (internal).
//
// A wave accumulates, for TR tiles of 16 weight rows and MT tiles of 16
// activation rows, the partial dot products over K steps [s0, s1) of 256
// elements.  Lane (n = lane % 16, q = lane / 16) loads, per step and weight
// tile, two 16-byte code words of its weight row -- elements [32q, 32q+32) and
// [128+32q, 160+32q) of the step -- plus the two scale bytes of each.  Each
// 32-bit word (8 elements sharing one scale) is decoded exactly to bf16 and is
// the B operand of one v_mfma_f32_16x16x32_bf16; the A operand carries the
// matching 8 activations of activation row (lane % 16) of the m-tile.
// Result layout (per tile pair): lane holds C[m = 4*(lane/16) + r][n = lane%16].
#pragma once

#include "device.h"

namespace nvfp4 {

constexpr int kGemvStep = 256;  // K elements per step

__device__ __forceinline__ u32x4 load16_or_zero(const uint8_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// xrow[mt]: this lane's activation row (bf16, K elements) for m-tile mt, or
// nullptr for a padding row.  cptr/sptr: this lane's weight-row code and scale
// pointers per weight tile; rvalid false for padding rows.
template <int MT, int TR>
__device__ __forceinline__ void gemv_accumulate(f32x4 (&acc)[TR][MT],
                                                const uint16_t* const (&xrow)[MT],
                                                const uint8_t* const (&cptr)[TR],
                                                const uint8_t* const (&sptr)[TR],
                                                const bool (&rvalid)[TR], int64_t K, int s0,
                                                int s1) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  for (int s = s0; s < s1; ++s) {
    const int64_t kb = (int64_t)s * kGemvStep;
    const int64_t k0 = kb + 32 * q, k1 = kb + 128 + 32 * q;
    const bool ok0 = k0 + 32 <= K, ok1 = k1 + 32 <= K;

    u32x4 xa[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bool mok = xrow[mt] != nullptr;
      const uint8_t* xr = mok ? reinterpret_cast<const uint8_t*>(xrow[mt]) : cptr[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xa[mt][j] = load16_or_zero(xr + (k0 + 8 * j) * 2, mok && ok0);
        xa[mt][4 + j] = load16_or_zero(xr + (k1 + 8 * j) * 2, mok && ok1);
      }
    }

#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const bool v0 = rvalid[t] && ok0, v1 = rvalid[t] && ok1;
      const u32x4 c0 = load16_or_zero(cptr[t] + k0 / 2, v0);
      const u32x4 c1 = load16_or_zero(cptr[t] + k1 / 2, v1);
      const uint32_t sc0 = v0 ? *reinterpret_cast<const uint16_t*>(sptr[t] + k0 / 16) : 0u;
      const uint32_t sc1 = v1 ? *reinterpret_cast<const uint16_t*>(sptr[t] + k1 / 16) : 0u;
      const float f00 = e4m3_to_f32<0>(sc0), f01 = e4m3_to_f32<1>(sc0);
      const float f10 = e4m3_to_f32<0>(sc1), f11 = e4m3_to_f32<1>(sc1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t cw = j < 4 ? c0[j] : c1[j - 4];
        const float sf = j < 2 ? f00 : j < 4 ? f01 : j < 6 ? f10 : f11;
        const u32x4 b = dequant8_bf16(cw, sf);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = mfma_16x16x32_bf16(xa[mt][j], b, acc[t][mt]);
      }
    }
  }
}

// Sum one f32x4 accumulator over the nw waves of the workgroup in wave order.
// Returns, for threads 0..255, the total of element r = tid/64 of lane tid%64
// (i.e. C[4*((tid%64)/16) + tid/64][tid%16]); other threads get 0.  `red` is
// nw*256 floats of LDS.  Contains two barriers; every thread must call it.
__device__ __forceinline__ float wave_sum_f32x4(float* red, const f32x4& v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  *reinterpret_cast<f32x4*>(&red[(wave * 64 + lane) * 4]) = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x < 256) {
    const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int w = 0; w < nw; ++w) s += red[(w * 64 + l) * 4 + r];
  }
  __syncthreads();
  return s;
}

}  // namespace nvfp4
