// gemm.hip -- prefill-shaped NVFP4 linear layer (large M) for gfx950.
//
// y = a . W^T with W = e2m1(code) * e4m3(scale) (NVFP4: "Serving Qwen3.8-27B in
// 4-bit with a masked speculative decoding head", section "What the artifact
// is"), bf16 activations (W4A16: "What 350+ Experiments Taught Us About Serving
// Qwen 3.6 35B-A3B", section 1) or NVFP4 activations (W4A4: "52.6% more
// tokens, 1.53x less GPU time: production inference with Minima and Rafay"),
// fp32 accumulation.  At M in the thousands every weight is reused M times, so
// the kernel is bound by the bf16 MFMA rate, not by HBM.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile of y; each wave a
// 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.  K advances
// 64 elements per step through a double buffer in LDS:
//   A tile  [256 rows][64] bf16 (32 KB): 16-byte pieces copied from global;
//   B tile  [256 cols][64] bf16 (32 KB): each thread loads one weight row's
//           32 code bytes and 4 scale bytes and writes the 64 exactly
//           dequantized bf16 values (the NVFP4 decode is done once per tile,
//           not per use).  NVFP4 activations are decoded the same way.
// Rows are stored as eight 16-byte pieces with piece c of row r at position
// c ^ (r & 7), so the 32 lanes of an MFMA operand read (rows r..r+31, the same
// piece) hit distinct LDS banks.
//
// Pipeline: the global loads of step s+2 are issued at the start of step s
// into one of two register sets; the other set (step s+1, loaded a whole step
// earlier) is decoded and written to the idle LDS buffer in four parts, one per
// 16-element substep, between the MFMAs of step s; one barrier per step.  Each
// substep's MFMA fragments are read from LDS while the previous substep's
// MFMAs run.
//
// The weight tile is the MFMA's A operand and the activation tile its B
// operand, so an accumulator block holds y^T: lane l has output row l % 32 and
// 4 consecutive output columns per register group, stored as one 8-byte (bf16)
// or 16-byte (fp32) write.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so each XCD is given a contiguous band of the tile sequence, which runs
// over n fastest within groups of 8 m-tiles; the tiles an XCD holds at once
// share activation rows and weight columns in its L2.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileElems = BM * BK;  // one bf16 operand tile in LDS

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

__device__ __forceinline__ int swz(int row, int piece) { return row * BK + ((piece ^ (row & 7)) << 3); }

// A thread's share of one step's global loads, exactly as loaded: every load
// is unconditional (addresses clamped into the arrays); the bytes past a
// partial last step (K % 64 == 32) are replaced by zeros when the set is
// written to LDS, so no wait for the loads is needed before then.
template <bool A_NVFP4>
struct GemmLoad {
  u32x4 a[A_NVFP4 ? 2 : 8];  // bf16: 8 pieces of 16 B; NVFP4: one row's 32 code bytes
  uint32_t a_sc[2];          // NVFP4: the row's 4 scale bytes as two 16-bit loads
  u32x4 w[2];                // one weight row's 32 code bytes
  uint32_t w_sc[2];          // its 4 scale bytes
};

template <bool A_NVFP4>
__device__ __forceinline__ void gemm_load(GemmLoad<A_NVFP4>& L, const GemmArgs& g, int64_t arow,
                                          int64_t wrow, int64_t k0) {
  const int t = threadIdx.x;
  const int64_t K = g.K;
  const bool kfull = k0 + BK <= K;
  const int hi = kfull ? 16 : 0;  // byte offset of the second code load (clamped)
  if constexpr (A_NVFP4) {
    const uint8_t* c = static_cast<const uint8_t*>(g.a) + arow * (K / 2) + k0 / 2;
    const uint16_t* s = reinterpret_cast<const uint16_t*>(g.a_scales + arow * (K / 16) + k0 / 16);
    L.a[0] = *reinterpret_cast<const u32x4*>(c);
    L.a[1] = *reinterpret_cast<const u32x4*>(c + hi);
    L.a_sc[0] = s[0];
    L.a_sc[1] = s[kfull ? 1 : 0];
  } else {
    // piece i of this thread: tile row t/8 + 32 i, piece t % 8
    const int p = t & 7;
    const int64_t k = k0 + 8 * p < K ? k0 + 8 * p : K - 8;
    const uint16_t* src = static_cast<const uint16_t*>(g.a) + arow * K + k;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t dm = min(arow + 32 * i, g.M - 1) - arow;  // rows past M repeat the last
      L.a[i] = *reinterpret_cast<const u32x4*>(src + dm * K);
    }
  }
  const uint8_t* c = g.wc + wrow * (K / 2) + k0 / 2;
  const uint16_t* s = reinterpret_cast<const uint16_t*>(g.ws + wrow * (K / 16) + k0 / 16);
  L.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c));
  L.w[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c + hi));
  L.w_sc[0] = s[0];
  L.w_sc[1] = s[kfull ? 1 : 0];
}

// Pieces 2q, 2q+1 (elements 16q .. 16q+15, one NVFP4 block) of one row ->
// exact bf16, written to the row's swizzled pieces.  A block at or past `kval`
// (the valid elements of the step, 0..64, a multiple of 32) gets scale 0: its
// codes were read from a clamped address inside the row and are finite, so it
// is written as zeros.
__device__ __forceinline__ void store_nvfp4_pieces(uint16_t* tile, int row, const u32x4 (&c)[2],
                                                   const uint32_t (&sc)[2], int q, int kval) {
  const uint32_t sw = sc[q >> 1];
  const float s_blk = (q & 1) ? e4m3_to_f32<1>(sw) : e4m3_to_f32<0>(sw);
  const float s = 16 * q < kval ? s_blk : 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = 2 * q + h;
    *reinterpret_cast<u32x4*>(tile + swz(row, p)) = dequant8_bf16(c[p >> 2][p & 3], s);
  }
}

// Part q (of 4) of writing a loaded set to LDS.
template <bool A_NVFP4>
__device__ __forceinline__ void gemm_store_part(const GemmLoad<A_NVFP4>& L, uint16_t* a_tile,
                                                uint16_t* b_tile, int q, int kval) {
  const int t = threadIdx.x;
  if constexpr (A_NVFP4) {
    store_nvfp4_pieces(a_tile, t, L.a, L.a_sc, q, kval);
  } else {
    const int p = t & 7;
    const bool live = 8 * p < kval;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * q + h;
      *reinterpret_cast<u32x4*>(a_tile + swz((t >> 3) + 32 * i, p)) = live ? L.a[i] : z;
    }
  }
  store_nvfp4_pieces(b_tile, t, L.w, L.w_sc, q, kval);
}

struct Frags {
  u32x4 w[4];  // weight rows (MFMA A operand), 4 blocks of 32
  u32x4 x[4];  // activation rows (MFMA B operand), 4 blocks of 32
};

// Operand layout (lane l): A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32],
// i.e. both read row l%32 of their tile block, piece 2*kk + l/32.
__device__ __forceinline__ void read_frags(Frags& f, const uint16_t* a_tile,
                                           const uint16_t* b_tile, int wm, int wn, int kk) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.x[i] = *reinterpret_cast<const u32x4*>(a_tile + swz(wm * 128 + i * 32 + r, 2 * kk + h));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.w[j] = *reinterpret_cast<const u32x4*>(b_tile + swz(wn * 128 + j * 32 + r, 2 * kk + h));
}

__device__ __forceinline__ void mfma_block(f32x16 (&acc)[4][4], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16_bf16(f.w[j], f.x[i], acc[i][j]);
}

// One 64-element step on LDS buffer `cur` while set L is written to buffer
// `nxt`.
template <bool A_NVFP4>
__device__ __forceinline__ void gemm_step(f32x16 (&acc)[4][4], const uint16_t* cur, uint16_t* nxt,
                                          const GemmLoad<A_NVFP4>& L, int kval, int wm, int wn) {
  Frags f0, f1;
  read_frags(f0, cur, cur + kTileElems, wm, wn, 0);
#pragma unroll
  for (int kk = 0; kk < 4; kk += 2) {
    read_frags(f1, cur, cur + kTileElems, wm, wn, kk + 1);
    gemm_store_part<A_NVFP4>(L, nxt, nxt + kTileElems, kk, kval);
    mfma_block(acc, f0);
    if (kk + 2 < 4) read_frags(f0, cur, cur + kTileElems, wm, wn, kk + 2);
    gemm_store_part<A_NVFP4>(L, nxt, nxt + kTileElems, kk + 1, kval);
    mfma_block(acc, f1);
  }
}

template <bool A_NVFP4>
__global__ void __launch_bounds__(kGemmThreads) k_gemm(GemmArgs g) {
  extern __shared__ uint16_t lds[];  // [2 buffers][A tile, B tile]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

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

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int64_t K = g.K;
  const int steps = (int)((K + BK - 1) / BK);
  const int steps2 = (steps + 1) & ~1;  // the loop runs step pairs; a padding step adds zeros
  // rows this thread loads: activation row (NVFP4: m0 + t; bf16: m0 + t/8, + 32 i)
  // and weight row `wrow` (into row t of the B tile)
  const int t = threadIdx.x;
  const int64_t arow = min(m0 + (A_NVFP4 ? t : (t >> 3)), g.M - 1);
  const int64_t n = min(n0 + (int64_t)t, g.N - 1);
  const int64_t wrow = g.row_idx ? (int64_t)g.row_idx[n] : n;
  // loads past the last step re-read it (their LDS copy is never used or is
  // zeroed through kval)
  auto kstep = [&](int s) -> int64_t { return (int64_t)(s < steps ? s : steps - 1) * BK; };
  auto kval = [&](int s) -> int {
    const int64_t v = K - (int64_t)s * BK;
    return v <= 0 ? 0 : (v >= BK ? BK : (int)v);
  };

  GemmLoad<A_NVFP4> L0, L1;
  gemm_load<A_NVFP4>(L0, g, arow, wrow, kstep(0));
  gemm_load<A_NVFP4>(L1, g, arow, wrow, kstep(1));
#pragma unroll
  for (int q = 0; q < 4; ++q) gemm_store_part<A_NVFP4>(L0, lds, lds + kTileElems, q, kval(0));
  __syncthreads();
  // At step s: buffer s&1 holds step s, set L[(s+1)&1] holds step s+1 (loaded
  // during step s-1) and set L[s&1] is free and takes step s+2.  The buffer
  // written during the last step is not read.
  uint16_t* b0 = lds;
  uint16_t* b1 = lds + 2 * kTileElems;
  // (the scheduling barriers keep each step's global loads at its start, a
  // whole step ahead of their use)
  for (int s = 0; s < steps2; s += 2) {
    gemm_load<A_NVFP4>(L0, g, arow, wrow, kstep(s + 2));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_NVFP4>(acc, b0, b1, L1, kval(s + 1), wm, wn);
    __syncthreads();
    gemm_load<A_NVFP4>(L1, g, arow, wrow, kstep(s + 3));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_NVFP4>(acc, b1, b0, L0, kval(s + 2), wm, wn);
    __syncthreads();
  }

  // acc[i][j] = y^T block (n-block j, m-block i): register e of lane l is output
  // row i*32 + l%32, column j*32 + 8*(e/4) + 4*(l/32) + e%4 of the wave's quarter.
  const int r = lane & 31, h = lane >> 5;
  const bool vec = (g.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + wm * 128 + i * 32 + r;
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * 128 + j * 32 + 8 * q + 4 * h;
        const int64_t o = row * g.N + col;
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (vec && col + 3 < g.N) {
          if (g.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + o) = f32x4{v0, v1, v2, v3};
          } else {
            const u32x2 pk = {(uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16),
                              (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + o) = pk;
          }
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= g.N) break;
            if (g.out_f32)
              static_cast<float*>(g.out)[o + e] = v[e];
            else
              static_cast<uint16_t*>(g.out)[o + e] = (uint16_t)f32_to_bf16_bits(v[e]);
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
  const size_t lds = 2 * 2 * (size_t)kTileElems * sizeof(uint16_t);
  if (a_nvfp4)
    hipLaunchKernelGGL(k_gemm<true>, dim3(grid), dim3(kGemmThreads), lds, stream, g);
  else
    hipLaunchKernelGGL(k_gemm<false>, dim3(grid), dim3(kGemmThreads), lds, stream, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
