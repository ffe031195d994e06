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
// 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (accumulators
// in AGPRs).  K advances 64 elements per step through a double buffer in LDS:
//   A tile  [256 rows][64] bf16 (32 KB): 16-byte pieces copied from global;
//   B tile  [256 cols][64] bf16 (32 KB): NVFP4 weight rows decoded exactly to
//           bf16 as they are written (once per tile, not per use).  NVFP4
//           activations are decoded the same way into the A tile.
// LDS layout: [A buffer 0][A buffer 1][B buffer 0][B buffer 1], so every LDS
// access is a per-lane base register plus an immediate offset.  Rows are eight
// 16-byte pieces, piece c of row r at c ^ f(r), f(r) = (r ^ (r >> 3)) & 7: the
// 16 consecutive rows of an MFMA operand read or of a tile write fall on
// distinct banks.
//
// Global loads: the bf16 activation tile is read 8 rows x 128 bytes per load
// instruction; NVFP4 rows cooperatively, two lanes per row (one 16-byte half
// each), so a load instruction touches 32 cache lines and every line is looked
// up once per step -- the line count per instruction, not bandwidth, is what
// these loads cost.
//
// Pipeline: the global loads of step s+2 are issued at the start of step s
// into one of two register sets; the other set (step s+1, loaded a whole step
// earlier) is decoded and written to the idle LDS buffers while step s is
// computed.  A step is 16 chunks (substep kk = 0..3, accumulator row i =
// 0..3): chunk (kk, i) issues the 4 MFMAs of row i, reads fragments x[i], w[i]
// of substep kk+1 and writes one 16-byte piece of the next tile; scheduling
// barriers keep that interleave.  One workgroup barrier per step.
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
constexpr uint32_t kTileBytes = BM * BK * 2;  // one bf16 operand tile (32 KB)
constexpr uint32_t kBOffset = 2 * kTileBytes;  // B buffers follow both A buffers
constexpr uint32_t kLdsBytes = 4 * kTileBytes;

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

__device__ __forceinline__ uint32_t swz_f(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

template <typename T>
__device__ __forceinline__ T& lds_ref(char* lds, uint32_t off) {
  return *reinterpret_cast<T*>(lds + off);
}

// Per-lane LDS byte offsets.  With r = lane % 32, h = lane / 32 and
// g = h ^ f(r): fragment (substep kk, block i) of the wave's activation rows
// wm*128 + 32 i + r sits at piece (2kk + h) ^ f(row) = 2 (kk ^ 2(i&1)) ^ g, so
// it is rd_x[kk ^ 2(i&1)] + 32 KB * buffer + 4096 i (likewise rd_w for the
// weight rows wn*128 + ...).  An NVFP4 row
// write (row t/2 + 128 q, piece 4 (t&1) + j) is wr_w[j] (weights) or wr_na[j]
// (NVFP4 activations) + 32 KB * buffer + 16384 q.  (Immediate offsets of LDS
// instructions stop at 64 KB, so the B-tile base is part of the registers.)
struct LdsOffsets {
  uint32_t rd_x[4], rd_w[4];
  uint32_t wr_w[4], wr_na[4];
};

__device__ __forceinline__ LdsOffsets lds_offsets(int wm, int wn) {
  LdsOffsets o;
  const uint32_t t = threadIdx.x, lane = t & 63, r = lane & 31, h = lane >> 5;
  const uint32_t g = (h ^ swz_f(r)) & 7u;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    o.rd_x[kk] = (wm * 128 + r) * 128 + (((2u * kk) ^ g) << 4);
    o.rd_w[kk] = kBOffset + (wn * 128 + r) * 128 + (((2u * kk) ^ g) << 4);
  }
  const uint32_t fw = ((t >> 1) ^ (t >> 4)) & 7u, hh = t & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o.wr_na[j] = (t >> 1) * 128 + (((4u * hh + j) ^ fw) << 4);
    o.wr_w[j] = kBOffset + o.wr_na[j];
  }
  return o;
}

// A thread's share of one step's global loads, exactly as loaded.  Every load
// is unconditional: on a partial last step (K % 64 == 32) the missing half is
// re-read from inside the row and zeroed when the set is written to LDS, so no
// wait for the loads is needed before then.
struct Nvfp4Rows {
  u32x4 c[2];     // codes of half (t & 1) of tile rows t/2 and 128 + t/2
  uint32_t s[2];  // their two E4M3 scale bytes (one 16-bit load each)
};
template <bool A_NVFP4>
struct GemmLoad;
template <>
struct GemmLoad<false> {
  Nvfp4Rows w;  // bf16 activations go to LDS directly (dma_a_tile)
};
template <>
struct GemmLoad<true> {
  Nvfp4Rows a;
  Nvfp4Rows w;
};

// Where a thread loads from: bf16 activations as byte offsets (32-bit) from
// the tile's first row at k = 0 (see dma_a_tile); NVFP4 rows as pointers to
// this lane's half of rows t/2 and 128 + t/2 at k = 0.
struct GemmSrc {
  uint32_t a_off[8];
  uint32_t a_back[2];
  const uint8_t* ac[2];
  const uint8_t* as[2];
  const uint8_t* wc[2];
  const uint8_t* ws[2];
};

__device__ __forceinline__ void load_nvfp4_rows(Nvfp4Rows& R, const uint8_t* const (&c)[2],
                                                const uint8_t* const (&s)[2], int64_t k0,
                                                bool kfull) {
  const int hh = threadIdx.x & 1;
  const int64_t coff = k0 / 2 - (kfull ? 0 : 16 * hh);
  const int64_t soff = k0 / 16 - (kfull ? 0 : 2 * hh);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    R.c[q] = *reinterpret_cast<const u32x4*>(c[q] + coff);
    R.s[q] = *reinterpret_cast<const uint16_t*>(s[q] + soff);
  }
}

template <bool A_NVFP4>
__device__ __forceinline__ void gemm_load(GemmLoad<A_NVFP4>& L, const GemmSrc& src,
                                          const uint8_t* a_tile_base, int64_t K, int64_t k0) {
  const bool kfull = k0 + BK <= K;
  if constexpr (A_NVFP4) load_nvfp4_rows(L.a, src.ac, src.as, k0, kfull);
  load_nvfp4_rows(L.w, src.wc, src.ws, k0, kfull);
}

// bf16 activation tile of the step at k0 -> LDS A buffer at `dst`, straight
// from global memory (global_load_lds_dwordx4: lane l of a load lands at the
// wave's LDS base + 16 l).  Wave w fills rows 64 w .. 64 w + 63, eight rows
// (1 KB of LDS) per load; lane l takes row 8 i + l/8 of its band and physical
// piece l % 8, i.e. logical piece (l % 8) ^ f(row) = (l % 8) ^ (l / 8) ^ i.
// On a partial last step (K % 64 == 32) logical pieces 4..7 re-read pieces
// 0..3: those k have zero weights, so the products vanish.
__device__ __forceinline__ void dma_a_tile(char* dst, const GemmSrc& src,
                                           const uint8_t* a_tile_base, int64_t k0, bool kfull) {
  const uint8_t* base = a_tile_base + 2 * k0;
  const int wave = threadIdx.x >> 6;
  const uint32_t keep = kfull ? 0u : ~0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint8_t* gp = base + (src.a_off[i] - (src.a_back[(i >> 2) & 1] & keep));
    __builtin_amdgcn_global_load_lds(gp, dst + (64 * wave + 8 * i) * 128, 16, 0, 0);
  }
}

// Piece j (0..3) of this thread's half of NVFP4 tile row t/2 + 128 q -> 8
// exact bf16 values.  A block at or past `kval` (the valid elements of the
// step, 0..64, a multiple of 32) gets scale 0; its codes are finite, so it is
// written as zeros.
__device__ __forceinline__ void store_nvfp4_piece(char* lds, uint32_t off, const Nvfp4Rows& R,
                                                  int q, int j, int kval) {
  const int p = 4 * (threadIdx.x & 1) + j;
  const float s_blk = (j >> 1) ? e4m3_to_f32<1>(R.s[q]) : e4m3_to_f32<0>(R.s[q]);
  const float s = 16 * (p >> 1) < kval ? s_blk : 0.f;
  lds_ref<u32x4>(lds, off) = dequant8_bf16(R.c[q][j], s);
}

// Piece c of writing a loaded set to LDS buffer `buf`: weight pieces 0..7,
// then (NVFP4 activations only) activation pieces 8..15.
template <bool A_NVFP4>
__device__ __forceinline__ void gemm_store_piece(char* lds, const LdsOffsets& o, uint32_t buf,
                                                 const GemmLoad<A_NVFP4>& L, int c, int kval) {
  const int q = (c & 7) >> 2, j = c & 3;
  if (c < 8) {
    store_nvfp4_piece(lds, o.wr_w[j] + buf * kTileBytes + q * 16384, L.w, q, j, kval);
  } else if constexpr (A_NVFP4) {
    store_nvfp4_piece(lds, o.wr_na[j] + buf * kTileBytes + q * 16384, L.a, q, j, kval);
  }
}

struct Frags {
  u32x4 w[4];  // weight rows (MFMA A operand), 4 blocks of 32
  u32x4 x[4];  // activation rows (MFMA B operand), 4 blocks of 32
};

// Operand layout (lane l): A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32],
// i.e. both read row l%32 of their tile block, piece 2*kk + l/32 (substep kk).
__device__ __forceinline__ void read_frag(Frags& f, char* lds, const LdsOffsets& o, uint32_t buf,
                                          int kk, int i) {
  const int kq = kk ^ (2 * (i & 1));
  f.x[i] = lds_ref<const u32x4>(lds, o.rd_x[kq] + buf * kTileBytes + i * 4096);
  f.w[i] = lds_ref<const u32x4>(lds, o.rd_w[kq] + buf * kTileBytes + i * 4096);
}

// One 64-element step on LDS buffer `cur` while set L is decoded into buffer
// `nxt`.  On entry f[0] holds the step's substep-0 fragments; substeps 0..2
// read the fragments of the next substep and write the pieces of the next
// tile; then the workgroup barrier publishes `nxt`, and substep 3 reads the
// next step's substep-0 fragments from it into f[0] while its MFMAs run, so no
// fragment read is left exposed behind the barrier.
template <bool A_NVFP4>
__device__ __forceinline__ void gemm_step(f32x16 (&acc)[4][4], Frags (&f)[2], char* lds,
                                          const LdsOffsets& o, uint32_t cur, uint32_t nxt,
                                          const GemmLoad<A_NVFP4>& L, int kval) {
  constexpr int kPieces = A_NVFP4 ? 16 : 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk == 3) lds_barrier<A_NVFP4 ? -1 : 0>();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kk < 3)
        read_frag(f[(kk + 1) & 1], lds, o, cur, kk + 1, i);
      else
        read_frag(f[0], lds, o, nxt, 0, i);
      const int c = 4 * kk + i;  // chunk 0..11 carries pieces c and c + 12
      if (kk < 3) {
        if (c < kPieces) gemm_store_piece<A_NVFP4>(lds, o, nxt, L, c, kval);
        if (c + 12 < kPieces) gemm_store_piece<A_NVFP4>(lds, o, nxt, L, c + 12, kval);
      }
      const Frags& fc = f[kk & 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16_bf16(fc.w[j], fc.x[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <bool A_NVFP4>
__global__ void __launch_bounds__(kGemmThreads) k_gemm(GemmArgs g) {
  extern __shared__ char lds[];
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
  const int t = threadIdx.x;

  // sources (rows past M or N are clamped to the last one; never stored)
  GemmSrc src;
  const uint8_t* a_tile_base = static_cast<const uint8_t*>(g.a) + (A_NVFP4 ? 0 : m0 * K * 2);
  const int hh = t & 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t n = min(n0 + (t >> 1) + 128 * q, g.N - 1);
    const int64_t wr = g.row_idx ? (int64_t)g.row_idx[n] : n;
    src.wc[q] = g.wc + wr * (K / 2) + 16 * hh;
    src.ws[q] = g.ws + wr * (K / 16) + 2 * hh;
    const int64_t ar = min(m0 + (t >> 1) + 128 * q, g.M - 1);
    src.ac[q] = static_cast<const uint8_t*>(g.a) + ar * (K / 2) + 16 * hh;
    src.as[q] = g.a_scales + ar * (K / 16) + 2 * hh;
  }
  {
    const int lw = t & 63, band = 64 * (t >> 6);
    const uint32_t lp = (uint32_t)((lw & 7) ^ (lw >> 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t dm = min(m0 + band + 8 * i + (lw >> 3), g.M - 1) - m0;
      src.a_off[i] = (uint32_t)((dm * K + 8 * ((lp ^ i) & 7)) * 2);
    }
    // partial step: logical pieces 4..7 step back 32 elements (bit 2 of lp ^ i)
    src.a_back[0] = (lp & 4) ? 64u : 0u;
    src.a_back[1] = (lp & 4) ? 0u : 64u;
  }
  const LdsOffsets o = lds_offsets(wm, wn);

  // loads past the last step re-read it (their LDS copy is never used or is
  // zeroed through kval)
  auto kstep = [&](int s) -> int64_t { return (int64_t)(s < steps ? s : steps - 1) * BK; };
  auto kval = [&](int s) -> int {
    const int64_t v = K - (int64_t)s * BK;
    return v <= 0 ? 0 : (v >= BK ? BK : (int)v);
  };

  // bf16 activations: the step's tile is copied into the next buffer during
  // the step before; each wave waits for its own copies before the barrier
  // that publishes the buffer.
  auto dma = [&](int s, uint32_t buf) {
    if constexpr (!A_NVFP4)
      dma_a_tile(lds + buf * kTileBytes, src, a_tile_base, kstep(s), kstep(s) + BK <= K);
  };

  GemmLoad<A_NVFP4> L0, L1;
  Frags f[2];
  dma(0, 0);
  gemm_load<A_NVFP4>(L0, src, a_tile_base, K, kstep(0));
  gemm_load<A_NVFP4>(L1, src, a_tile_base, K, kstep(1));
#pragma unroll
  for (int c = 0; c < 16; ++c) gemm_store_piece<A_NVFP4>(lds, o, 0, L0, c, kval(0));
  lds_barrier<A_NVFP4 ? -1 : 0>();
#pragma unroll
  for (int i = 0; i < 4; ++i) read_frag(f[0], lds, o, 0, 0, i);
  // At step s: buffer s&1 holds step s, set L[(s+1)&1] holds step s+1 (loaded
  // during step s-1) and set L[s&1] is free and takes step s+2.  The buffer
  // written during the last step is not read.  The scheduling barriers keep
  // each step's global loads at its start, ahead of their use.
  for (int s = 0; s < steps2; s += 2) {
    dma(s + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load<A_NVFP4>(L0, src, a_tile_base, K, kstep(s + 2));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_NVFP4>(acc, f, lds, o, 0, 1, L1, kval(s + 1));
    dma(s + 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load<A_NVFP4>(L1, src, a_tile_base, K, kstep(s + 3));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_NVFP4>(acc, f, lds, o, 1, 0, L0, kval(s + 2));
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
