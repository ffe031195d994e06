// gemm.hip -- prefill-shaped NVFP4 linear layer (large M) for gfx950.
//
// y = a . W^T with W = e2m1(code) * e4m3(scale) (NVFP4: "Serving Qwen3.8-27B in
// 4-bit with a masked speculative decoding head", section "What the artifact
// is"), bf16 activations (W4A16: "What 350+ Experiments Taught Us About Serving
// Qwen 3.6 35B-A3B", section 1) or NVFP4 activations (W4A4: "52.6% more
// tokens, 1.53x less GPU time: production inference with Minima and Rafay"),
// fp32 accumulation.  At M in the thousands every weight is reused M times, so
// the kernel is bound by the bf16 MFMA rate, not by HBM.  The 256 x 256 tile
// is gemm_core.h.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so each XCD is given a contiguous band of the tile sequence, which runs
// over n fastest within groups of 8 m-tiles; the tiles an XCD holds at once
// share activation rows and weight columns in its L2.
#include "gemm_core.h"
#include "launch.h"

namespace nvfp4 {

namespace {

struct GemmArgs {
  const void* a;            // bf16 [M][K], or NVFP4 codes [M][K/2]
  const uint8_t* a_scales;  // NVFP4 activations: [M][K/16]
  const uint8_t* wc;        // weight codes [rows][K/2]
  const uint8_t* ws;        // weight scales [rows][K/16]
  const int32_t* row_idx;   // output column n uses weight row row_idx[n]; null: row n
  void* out;                // [M][N] bf16 or fp32
  int64_t M, N, K;          // N: output columns
  int out_f32;
  int tiles_m, tiles_n;
};

template <bool A_NVFP4>
__global__ void __launch_bounds__(kGemmThreads) k_gemm(GemmArgs g) {
  extern __shared__ char lds[];

  const int total = g.tiles_m * g.tiles_n;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  constexpr int GM = 8;
  const int group = lin / (GM * g.tiles_n);
  const int gm0 = group * GM;
  const int gsz = min(GM, g.tiles_m - gm0);
  const int in_group = lin - group * GM * g.tiles_n;
  const int tm = gm0 + in_group % gsz, tn = in_group / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t K = g.K;
  const int t = threadIdx.x;

  // sources (rows past M or N are clamped to the last one; never stored)
  GemmSrc src;
  const uint8_t* a_tile_base = static_cast<const uint8_t*>(g.a) + (A_NVFP4 ? 0 : m0 * K * 2);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t n = min(n0 + (t >> 1) + 128 * q, g.N - 1);
    const int64_t wr = g.row_idx ? (int64_t)g.row_idx[n] : n;
    gemm_src_nvfp4_row(src.wc[q], src.ws[q], g.wc, g.ws, wr, K);
    if constexpr (A_NVFP4) {
      const int64_t ar = min(m0 + (t >> 1) + 128 * q, g.M - 1);
      gemm_src_nvfp4_row(src.ac[q], src.as[q], static_cast<const uint8_t*>(g.a), g.a_scales, ar,
                         K);
    }
  }
  if constexpr (!A_NVFP4)
    gemm_src_bf16(src, [&](int r) { return min(m0 + r, g.M - 1) - m0; }, K);

  f32x16 acc[4][4];
  gemm_zero_acc(acc);
  gemm_mainloop<A_NVFP4>(acc, lds, src, a_tile_base, K);

  // acc[i][j] = y^T block (n-block j, m-block i): register e of lane l is output
  // row i*32 + l%32, column j*32 + 8*(e/4) + 4*(l/32) + e%4 of the wave's quarter.
  const bool vec = (g.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + gemm_tile_row(i);
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + gemm_tile_col(j, q);
        const int64_t off = row * g.N + col;
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (vec && col + 3 < g.N) {
          if (g.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + off) = f32x4{v0, v1, v2, v3};
          } else {
            const u32x2 pk = {(uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16),
                              (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + off) = pk;
          }
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= g.N) break;
            if (g.out_f32)
              static_cast<float*>(g.out)[off + e] = v[e];
            else
              static_cast<uint16_t*>(g.out)[off + e] = (uint16_t)f32_to_bf16_bits(v[e]);
          }
        }
      }
    }
  }
}

}  // namespace

int launch_gemm(bool a_nvfp4, const void* a, const uint8_t* a_scales, int64_t M, int64_t K,
                const uint8_t* wc, const uint8_t* ws, const int32_t* row_idx, int64_t n_out,
                bool out_f32, void* out, hipStream_t stream) {
  // activation offsets inside a 256-row tile are 32-bit byte offsets
  if (K > ((int64_t)1 << 22)) return -1;
  GemmArgs g;
  g.a = a;
  g.a_scales = a_scales;
  g.wc = wc;
  g.ws = ws;
  g.row_idx = row_idx;
  g.out = out;
  g.M = M;
  g.N = n_out;
  g.K = K;
  g.out_f32 = out_f32 ? 1 : 0;
  g.tiles_m = (int)((M + BM - 1) / BM);
  g.tiles_n = (int)((n_out + BN - 1) / BN);
  const int total = g.tiles_m * g.tiles_n;
  const int grid = ((total + 7) / 8) * 8;
  if (a_nvfp4)
    hipLaunchKernelGGL(k_gemm<true>, dim3(grid), dim3(kGemmThreads), kLdsBytes, stream, g);
  else
    hipLaunchKernelGGL(k_gemm<false>, dim3(grid), dim3(kGemmThreads), kLdsBytes, stream, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
