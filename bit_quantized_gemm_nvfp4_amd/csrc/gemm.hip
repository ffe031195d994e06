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
  float* partial;           // splits > 1: fp32 [splits][M][N]
  int64_t M, N, K;          // N: output columns
  int64_t k_split;          // K elements per split (a multiple of 64; the last may be shorter)
  int out_f32;
  int tiles_m, tiles_n;
  int splits;               // split-K parts (1: no split)
  const float* ga;          // two-level scales: final sums are multiplied by
  const float* gw;          // *ga * *gw (null: 1)
};

template <bool A_NVFP4>
__global__ void __launch_bounds__(kGemmThreads) k_gemm(GemmArgs g) {
  extern __shared__ char lds[];

  const int tiles = g.tiles_m * g.tiles_n;
  const int total = tiles * g.splits;
  const int per_xcd = (total + 7) / 8;
  const int lin_all = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin_all >= total) return;
  const int z = lin_all / tiles, lin = lin_all - z * tiles;  // split z of tile `lin`
  constexpr int GM = 8;
  const int group = lin / (GM * g.tiles_n);
  const int gm0 = group * GM;
  const int gsz = min(GM, g.tiles_m - gm0);
  const int in_group = lin - group * GM * g.tiles_n;
  const int tm = gm0 + in_group % gsz, tn = in_group / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t K = g.K;
  const int64_t k_lo = (int64_t)z * g.k_split;
  const int64_t k_len = min(g.k_split, K - k_lo);
  const int t = threadIdx.x;

  // sources (rows past M or N are clamped to the last one; never stored)
  GemmSrc src;
  // (K ranges of a split start at k_lo: a multiple of 64, so pointers stay aligned)
  const uint8_t* a_tile_base =
      static_cast<const uint8_t*>(g.a) + (A_NVFP4 ? 0 : m0 * K * 2 + 2 * k_lo);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t n = min(n0 + (t >> 1) + 128 * q, g.N - 1);
    const int64_t wr = g.row_idx ? (int64_t)g.row_idx[n] : n;
    gemm_src_nvfp4_row(src.wc[q], src.ws[q], g.wc + k_lo / 2, g.ws + k_lo / 16, wr, K);
    if constexpr (A_NVFP4) {
      const int64_t ar = min(m0 + (t >> 1) + 128 * q, g.M - 1);
      gemm_src_nvfp4_row(src.ac[q], src.as[q], static_cast<const uint8_t*>(g.a) + k_lo / 2,
                         g.a_scales + k_lo / 16, ar, K);
    }
  }
  if constexpr (!A_NVFP4)
    gemm_src_bf16(src, [&](int r) { return min(m0 + r, g.M - 1) - m0; }, K);

  f32x16 acc[4][4];
  gemm_zero_acc(acc);
  gemm_mainloop<A_NVFP4>(acc, lds, src, a_tile_base, k_len);

  // split z > 0 or any split of a split-K launch: fp32 partials
  const bool part = g.splits > 1;
  void* const dst = part ? static_cast<void*>(g.partial + (int64_t)z * g.M * g.N) : g.out;
  const bool f32 = part || g.out_f32;
  const bool scaled = !part && (g.ga || g.gw);
  const float alpha = scaled ? alpha_of(g.ga, g.gw) : 1.0f;

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
        float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (scaled) v0 *= alpha, v1 *= alpha, v2 *= alpha, v3 *= alpha;
        if (vec && col + 3 < g.N) {
          if (f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + off) = f32x4{v0, v1, v2, v3};
          } else {
            const u32x2 pk = {(uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16),
                              (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + off) = pk;
          }
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= g.N) break;
            if (f32)
              static_cast<float*>(dst)[off + e] = v[e];
            else
              static_cast<uint16_t*>(dst)[off + e] = (uint16_t)f32_to_bf16_bits(v[e]);
          }
        }
      }
    }
  }
}

// Split-K sum: out = sum over splits (in split order) of the fp32 partials.
__global__ void __launch_bounds__(256) k_gemm_reduce(const float* __restrict__ partial,
                                                     int splits, int64_t count, int out_f32,
                                                     const float* ga, const float* gw,
                                                     void* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= count) return;
  const bool scaled = ga || gw;
  const float alpha = scaled ? alpha_of(ga, gw) : 1.0f;
  if (i + 4 <= count) {
    f32x4 v = *reinterpret_cast<const f32x4*>(partial + i);
    for (int z = 1; z < splits; ++z) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(partial + (int64_t)z * count + i);
      v[0] += p[0], v[1] += p[1], v[2] += p[2], v[3] += p[3];
    }
    if (scaled) v[0] *= alpha, v[1] *= alpha, v[2] *= alpha, v[3] *= alpha;
    if (out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = v;
    } else {
      const u32x2 pk = {(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                        (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i) = pk;
    }
    return;
  }
  for (int64_t j = i; j < count; ++j) {
    float v = partial[j];
    for (int z = 1; z < splits; ++z) v += partial[(int64_t)z * count + j];
    if (scaled) v *= alpha;
    if (out_f32)
      static_cast<float*>(out)[j] = v;
    else
      static_cast<uint16_t*>(out)[j] = f32_to_bf16_bits(v);
  }
}

}  // namespace

int gemm_splits(int64_t M, int64_t n_out, int64_t K, int num_cus) {
  // One 256 x 256 tile per CU at a time (128 KB of LDS): with z splits the
  // compute takes rounds(z) = ceil(tiles * z / CUs) rounds of 1/z of K, and
  // the z fp32 partials are written and read once more.  Estimate both with
  // the measured rates (about 3.5 TFLOP/s per CU, 5 TB/s of HBM) and take the
  // cheapest z, keeping >= 8 steps (512 elements of K) per split.
  const int64_t tiles = ((M + BM - 1) / BM) * ((n_out + BN - 1) / BN);
  if (tiles >= num_cus) return 1;  // only a launch that cannot fill the chip once is split
  const int64_t steps = (K + BK - 1) / BK;
  const double round_s = 2.0 * BM * BN * (double)K / 3.5e12;
  const double part_s = (double)M * (double)n_out * 4.0 / 5.0e12;
  auto cost = [&](int64_t z) {
    const double rounds = (double)((tiles * z + num_cus - 1) / num_cus);
    return rounds * round_s / (double)z + (z > 1 ? (double)(z + 1) * part_s : 0.0);
  };
  int best = 1;
  for (int64_t z = 2; z <= 8 && z <= steps / 8; ++z)
    if (cost(z) < 0.95 * cost(best)) best = (int)z;
  return best;
}

size_t gemm_workspace_bytes(int64_t M, int64_t n_out, int64_t K, int num_cus) {
  const int z = gemm_splits(M, n_out, K, num_cus);
  return z > 1 ? (size_t)z * (size_t)M * (size_t)n_out * sizeof(float) : 0;
}

int launch_gemm(bool a_nvfp4, const void* a, const uint8_t* a_scales, int64_t M, int64_t K,
                const uint8_t* wc, const uint8_t* ws, const int32_t* row_idx, int64_t n_out,
                bool out_f32, void* out, void* workspace, hipStream_t stream, Alpha alpha) {
  // activation offsets inside a 256-row tile are 32-bit byte offsets
  if (K > ((int64_t)1 << 22)) return -1;
  GemmArgs g;
  g.ga = alpha.a;
  g.gw = alpha.w;
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
  g.splits = gemm_splits(M, n_out, K, kNumCUs);
  const int64_t steps = (K + BK - 1) / BK;
  g.k_split = ((steps + g.splits - 1) / g.splits) * BK;
  g.splits = (int)((K + g.k_split - 1) / g.k_split);  // every split non-empty
  g.partial = static_cast<float*>(workspace);
  if (g.splits > 1 && !workspace) return -1;
  const int total = g.tiles_m * g.tiles_n * g.splits;
  const int grid = ((total + 7) / 8) * 8;
  if (a_nvfp4)
    hipLaunchKernelGGL(k_gemm<true>, dim3(grid), dim3(kGemmThreads), kLdsBytes, stream, g);
  else
    hipLaunchKernelGGL(k_gemm<false>, dim3(grid), dim3(kGemmThreads), kLdsBytes, stream, g);
  if (hipGetLastError() != hipSuccess) return -1;
  if (g.splits > 1) {
    const int64_t count = M * n_out;
    const int64_t threads = (count + 3) / 4;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(workspace), g.splits, count, out_f32 ? 1 : 0,
                       alpha.a, alpha.w, out);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace nvfp4
