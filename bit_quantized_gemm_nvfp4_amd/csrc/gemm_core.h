// gemm_core.h -- the 256 x 256 MFMA tile of the NVFP4 GEMM kernels (internal):
// the large-M linear layer (gemm.hip) and the grouped expert GEMM (moe.hip).
//
// A workgroup of 8 waves (two per SIMD) computes a 256 x 256 tile of
// y = a . W^T; wave w a 128 (weight rows, wn = w & 1) x 64 (activation rows,
// wm = w >> 1) part as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (accumulators
// in AGPRs).  Two waves share each SIMD, so one wave's MFMAs keep the matrix
// core busy while the other waits on LDS, global loads or the barrier (with
// one 128 x 128 wave per SIMD, measured: MFMA busy 51%, 39% of wave cycles
// waiting).  K advances 64 elements per step through a double buffer in LDS:
//   A tile  [256 rows][64] bf16 (32 KB): bf16 activations copied global->LDS
//           (global_load_lds_dwordx4), or (A_FQ: the W4A4 product from bf16
//           activations) loaded through registers, quantized to NVFP4 and
//           dequantized exactly on the way;
//   B tile  [256 cols][64] bf16 (32 KB): NVFP4 weight rows decoded exactly to
//           bf16 as they are written (once per tile, not per use).
// LDS layout: [A buffer 0][A buffer 1][B buffer 0][B buffer 1], so every LDS
// access is a per-lane base register plus an immediate offset.  Rows are eight
// 16-byte pieces, piece c of row r at c ^ f(r), f(r) = (r ^ (r >> 3)) & 7: the
// 16 consecutive rows of an MFMA operand read or of a tile write fall on
// distinct banks.
//
// Global loads: the activation tile is copied 8 rows x 128 bytes per load
// instruction; NVFP4 rows are loaded cooperatively, two lanes per row (one
// 16-byte half each), so a load instruction touches 32 cache lines and every
// line is looked up once per step -- the line count per instruction, not
// bandwidth, is what these loads cost.  A_FQ activation rows are loaded the
// same way, two lanes per row, each lane 64 bytes (two whole 16-element
// blocks), so a block's maximum needs no exchange between lanes.
//
// Pipeline: the weight (and A_FQ activation) loads of step s+2 are issued at
// the start of step s into one of two register sets, the bf16 activation copy
// of step s+1 straight into the idle LDS buffer; the other register set (step
// s+1) is decoded into the idle buffer while step s is computed.  A step is 8
// chunks (substep kk = 0..3, activation block i = 0..1): chunk (kk, i) issues
// the 4 MFMAs of block i, reads fragments of substep kk+1 and writes pieces of
// the next tile; scheduling barriers keep that interleave.  One LDS-only
// workgroup barrier per step, between substeps 2 and 3.
//
// The weight tile is the MFMA's A operand and the activation tile its B
// operand, so an accumulator block holds y^T: lane l has output row l % 32 and
// 4 consecutive output columns per register group (gemm_tile_row/col).
#pragma once

#include "device.h"
#include "quant_core.h"

namespace nvfp4 {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 512;
constexpr int kXBlocks = 2;  // 32-row activation blocks per wave
constexpr int kWBlocks = 4;  // 32-row weight blocks per wave
constexpr uint32_t kTileBytes = BM * BK * 2;  // one bf16 operand tile (32 KB)
constexpr uint32_t kBOffset = 2 * kTileBytes;  // B buffers follow both A buffers
constexpr uint32_t kLdsBytes = 4 * kTileBytes;


__device__ __forceinline__ uint32_t swz_f(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

template <typename T>
__device__ __forceinline__ T& lds_ref(char* lds, uint32_t off) {
  return *reinterpret_cast<T*>(lds + off);
}

// Per-lane LDS byte offsets.  With r = lane % 32, h = lane / 32 and
// g = h ^ f(r): fragment (substep kk, block i) of the wave's activation rows
// wm*64 + 32 i + r sits at piece (2kk + h) ^ f(row) = 2 (kk ^ 2(i&1)) ^ g, so
// it is rd_x[kk ^ 2(i&1)] + 32 KB * buffer + 4096 i (likewise rd_w for the
// weight rows wn*128 + 32 j + r).  The row write of a thread's half (row t/2,
// piece 4 (t&1) + j) is wr_w[j] (weights) or wr_na[j] (A_FQ activations) +
// 32 KB * buffer.  (Immediate offsets of LDS instructions stop at 64 KB, so
// the B-tile base is part of the registers.)
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
    o.rd_x[kk] = (wm * 64 + r) * 128 + (((2u * kk) ^ g) << 4);
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
  u32x4 c;     // codes of half (t & 1) of tile row t/2
  uint32_t s;  // its two E4M3 scale bytes (one 16-bit load)
};
struct Bf16Rows {
  u32x4 v[4];  // half (t & 1) of tile row t/2: 32 bf16
};
template <bool A_FQ>
struct GemmLoad;
template <>
struct GemmLoad<false> {
  Nvfp4Rows w;  // bf16 activations go to LDS directly (dma_a_tile)
};
template <>
struct GemmLoad<true> {
  Bf16Rows a;
  Nvfp4Rows w;
};

// Where a thread loads from: bf16 activations as byte offsets (32-bit) from a
// base pointer at k = 0 (see dma_a_tile); its NVFP4 weight row as pointers to
// this lane's half of row t/2 at k = 0 (gemm_src_nvfp4_row); an A_FQ
// activation row as a pointer to this lane's half of row t/2.
//
// Weight addresses (TW: tiled weights).  Row-major: element k of the lane's
// row is at byte k / 2 of its codes and k / 16 of its scales.  Tiled
// (tile.hip): the 64 elements [k, k + 64) of a row (k a multiple of 64) are
// lane (row % 16, (k / 64) % 4) of block k / 256, so the codes of the lane's
// half sit at (k / 256) * 2304 + ((k / 64) % 4) * 256 from its pointer and
// the scales at (k / 256) * 2304 + ((k / 64) % 4) * 64.  k is
// workgroup-uniform, so on tiled weights the whole offset is scalar.
struct GemmSrc {
  uint32_t a_off[4];
  uint32_t a_back[4];
  const uint16_t* ar;
  const uint8_t* wc;  // this lane's codes and scales at k = 0 of its row
  const uint8_t* ws;
  int64_t k_lo;       // first element of the workgroup's K range
};

template <bool TW>
__device__ __forceinline__ void load_nvfp4_rows(Nvfp4Rows& R, const GemmSrc& src, int64_t k0,
                                                bool kfull) {
  const int64_t k = src.k_lo + k0;
  if constexpr (TW) {  // the layout pads K with zeros: no re-read on a partial step
    const int64_t blk = (k >> 8) * 2304, q = (k >> 6) & 3;
    R.c = *reinterpret_cast<const u32x4*>(src.wc + blk + 256 * q);
    R.s = *reinterpret_cast<const uint16_t*>(src.ws + blk + 64 * q);
  } else {
    const int hh = threadIdx.x & 1;
    const int64_t coff = k / 2 - (kfull ? 0 : 16 * hh);
    const int64_t soff = k / 16 - (kfull ? 0 : 2 * hh);
    R.c = *reinterpret_cast<const u32x4*>(src.wc + coff);
    R.s = *reinterpret_cast<const uint16_t*>(src.ws + soff);
  }
}

// A_FQ: 32 bf16 activations of this lane's half of its row (a partial last
// step re-reads the first half, as load_nvfp4_rows does).
__device__ __forceinline__ void load_bf16_rows(Bf16Rows& R, const uint16_t* a, int64_t k0,
                                               bool kfull) {
  const int hh = threadIdx.x & 1;
  const int64_t off = k0 - (kfull ? 0 : 32 * hh);
#pragma unroll
  for (int j = 0; j < 4; ++j) R.v[j] = *reinterpret_cast<const u32x4*>(a + off + 8 * j);
}

template <bool A_FQ, bool TW>
__device__ __forceinline__ void gemm_load(GemmLoad<A_FQ>& L, const GemmSrc& src,
                                          const uint8_t* a_tile_base, int64_t K, int64_t k0) {
  const bool kfull = k0 + BK <= K;
  if constexpr (A_FQ) load_bf16_rows(L.a, src.ar, k0, kfull);
  load_nvfp4_rows<TW>(L.w, src, k0, kfull);
}

// bf16 activation tile of the step at k0 -> LDS A buffer at `dst`, straight
// from global memory (global_load_lds_dwordx4: lane l of a load lands at the
// wave's LDS base + 16 l).  Wave w fills rows 32 w .. 32 w + 31, eight rows
// (1 KB of LDS) per load; lane l takes row 32 w + 8 i + l/8 and physical piece
// l % 8, i.e. logical piece (l % 8) ^ f(row) = (l % 8) ^ (l / 8) ^ ((4w + i) & 7).
// On a partial last step (K % 64 == 32) logical pieces 4..7 re-read pieces
// 0..3: those k have zero weights, so the products vanish.
__device__ __forceinline__ void dma_a_tile(char* dst, const GemmSrc& src,
                                           const uint8_t* a_tile_base, int64_t k0, bool kfull) {
  const uint8_t* base = a_tile_base + 2 * k0;
  const int wave = threadIdx.x >> 6;
  const uint32_t keep = kfull ? 0u : ~0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* gp = base + (src.a_off[i] - (src.a_back[i] & keep));
    __builtin_amdgcn_global_load_lds(gp, dst + (32 * wave + 8 * i) * 128, 16, 0, 0);
  }
}

// Piece j (0..3) of this thread's half of NVFP4 tile row t/2 -> 8 exact bf16
// values.  A block at or past `kval` (the valid elements of the step, 0..64, a
// multiple of 32) gets scale 0; its codes are finite, so it is written as
// zeros.
__device__ __forceinline__ void store_nvfp4_piece(char* lds, uint32_t off, const Nvfp4Rows& R,
                                                  int j, int kval) {
  const int p = 4 * (threadIdx.x & 1) + j;
  const float s_blk = (j >> 1) ? e4m3_to_f32<1>(R.s) : e4m3_to_f32<0>(R.s);
  const float s = 16 * (p >> 1) < kval ? s_blk : 0.f;
  lds_ref<u32x4>(lds, off) = dequant8_bf16(R.c[j], s);
}

// A_FQ: piece j (0..3) of this thread's half of activation tile row t/2,
// quantized to NVFP4 with its 16-element block (pieces j and j ^ 1, both in
// this lane) and dequantized: exactly nvfp4_quantize then nvfp4_dequantize.  A
// block at or past `kval` is written as zeros.
__device__ __forceinline__ void store_fq_piece(char* lds, uint32_t off, const Bf16Rows& R, int j,
                                               int kval) {
  const int p = 4 * (threadIdx.x & 1) + j;
  const u32x4 z = {0u, 0u, 0u, 0u};
  if (16 * (p >> 1) >= kval) {
    lds_ref<u32x4>(lds, off) = z;
    return;
  }
  const uint32_t amax = max(piece_amax_bits(R.v[j]), piece_amax_bits(R.v[j ^ 1]));
  lds_ref<u32x4>(lds, off) = fakequant_with(R.v[j], scale_code_from_amax(bf16_bits_to_f32(amax)));
}

// Piece c of writing a loaded set to LDS buffer `buf`: weight pieces 0..3,
// then (A_FQ only) activation pieces 4..7.
template <bool A_FQ>
__device__ __forceinline__ void gemm_store_piece(char* lds, const LdsOffsets& o, uint32_t buf,
                                                 const GemmLoad<A_FQ>& L, int c, int kval) {
  const int j = c & 3;
  if (c < 4) {
    store_nvfp4_piece(lds, o.wr_w[j] + buf * kTileBytes, L.w, j, kval);
  } else if constexpr (A_FQ) {
    store_fq_piece(lds, o.wr_na[j] + buf * kTileBytes, L.a, j, kval);
  }
}

struct Frags {
  u32x4 w[kWBlocks];  // weight rows (MFMA A operand), 4 blocks of 32
  u32x4 x[kXBlocks];  // activation rows (MFMA B operand), 2 blocks of 32
};

// Operand layout (lane l): A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32],
// i.e. both read row l%32 of their tile block, piece 2*kk + l/32 (substep kk).
__device__ __forceinline__ void read_x(Frags& f, char* lds, const LdsOffsets& o, uint32_t buf,
                                       int kk, int i) {
  f.x[i] = lds_ref<const u32x4>(lds, o.rd_x[kk ^ (2 * (i & 1))] + buf * kTileBytes + i * 4096);
}
__device__ __forceinline__ void read_w(Frags& f, char* lds, const LdsOffsets& o, uint32_t buf,
                                       int kk, int j) {
  f.w[j] = lds_ref<const u32x4>(lds, o.rd_w[kk ^ (2 * (j & 1))] + buf * kTileBytes + j * 4096);
}
// The fragments chunk i (0, 1) of a substep reads for its successor: x[i]
// (if block i is one of the wave's XL live activation blocks), w[2i],
// w[2i+1] (if any block is live).
template <int XL>
__device__ __forceinline__ void read_frag(Frags& f, char* lds, const LdsOffsets& o, uint32_t buf,
                                          int kk, int i) {
  if (i < XL) read_x(f, lds, o, buf, kk, i);
  if (XL > 0) {
    read_w(f, lds, o, buf, kk, 2 * i);
    read_w(f, lds, o, buf, kk, 2 * i + 1);
  }
}

// One 64-element step on LDS buffer `cur` while set L is decoded into buffer
// `nxt`.  On entry f[0] holds the step's substep-0 fragments; substeps 0..2
// read the fragments of the next substep and write the pieces of the next
// tile; then the workgroup barrier publishes `nxt`, and substep 3 reads the
// next step's substep-0 fragments from it into f[0] while its MFMAs run, so no
// fragment read is left exposed behind the barrier.  (Chunk i of a substep
// uses all four weight fragments of the substep: its successor's fragments
// go to the other set.)  XL: the wave's live activation blocks (2: all; 1:
// block 0 only; 0: none -- the wave only loads, decodes and meets the others);
// the MFMAs and operand reads of a dead block are skipped.
template <bool A_FQ, int XL>
__device__ __forceinline__ void gemm_step(f32x16 (&acc)[kXBlocks][kWBlocks], Frags (&f)[2],
                                          char* lds, const LdsOffsets& o, uint32_t cur,
                                          uint32_t nxt, const GemmLoad<A_FQ>& L, int kval) {
  constexpr int kPieces = A_FQ ? 8 : 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk == 3) lds_barrier<A_FQ ? -1 : 0>();
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i) {
      if (kk < 3)
        read_frag<XL>(f[(kk + 1) & 1], lds, o, cur, kk + 1, i);
      else
        read_frag<XL>(f[0], lds, o, nxt, 0, i);
      const int c = 2 * kk + i;  // chunk 0..5 carries pieces c and c + 6
      if (kk < 3) {
        if (c < kPieces) gemm_store_piece<A_FQ>(lds, o, nxt, L, c, kval);
        if (c + 6 < kPieces) gemm_store_piece<A_FQ>(lds, o, nxt, L, c + 6, kval);
      }
      if (i < XL) {
        const Frags& fc = f[kk & 1];
#pragma unroll
        for (int j = 0; j < kWBlocks; ++j)
          acc[i][j] = mfma_32x32x16_bf16(fc.w[j], fc.x[i], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The tile row of this thread's copy i (0..3) of a step's activation tile.
__device__ __forceinline__ int gemm_copy_row(int i) {
  return 32 * (threadIdx.x >> 6) + 8 * i + ((threadIdx.x & 63) >> 3);
}

// Sources of the tile's rows for this thread.  bf16 activation rows: the byte
// offsets (relative to the tile's base, k = 0) of this thread's four copies
// from their global rows r[i] (gemm_src_bf16_rows), or from abs_row(t), the
// global row (clamped to a valid one) of tile row t (gemm_src_bf16).  Weight
// and A_FQ activation rows: the pointer to this lane's half of the row at k =
// 0 (gemm_src_nvfp4_row).
__device__ __forceinline__ void gemm_src_bf16_rows(GemmSrc& src, const int64_t (&r)[4],
                                                   int64_t K) {
  const int t = threadIdx.x;
  const int lw = t & 63, wave = t >> 6;
  const uint32_t lp = (uint32_t)((lw & 7) ^ (lw >> 3));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t piece = (lp ^ (uint32_t)(4 * wave + i)) & 7u;  // logical piece
    src.a_off[i] = (uint32_t)((r[i] * K + 8 * piece) * 2);
    // partial step: logical pieces 4..7 step back 32 elements
    src.a_back[i] = (piece & 4) ? 64u : 0u;
  }
}

template <typename ARow>
__device__ __forceinline__ void gemm_src_bf16(GemmSrc& src, ARow abs_row, int64_t K) {
  int64_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = abs_row(gemm_copy_row(i));
  gemm_src_bf16_rows(src, r, K);
}

// This lane's pointers (its half of weight row `row`, k = 0), for a workgroup
// whose K range starts at k_lo.
__device__ __forceinline__ void gemm_src_nvfp4_row(GemmSrc& src, const uint8_t* codes,
                                                   const uint8_t* scales, int64_t row, int64_t K,
                                                   int64_t k_lo) {
  const int hh = threadIdx.x & 1;
  src.wc = codes + row * (K / 2) + 16 * hh;
  src.ws = scales + row * (K / 16) + 2 * hh;
  src.k_lo = k_lo;
}

// The same on tiled weights `wt` (ceil(K / 256) blocks per 16-row tile).
__device__ __forceinline__ void gemm_src_tiled_row(GemmSrc& src, const uint8_t* wt, int64_t row,
                                                   int64_t K, int64_t k_lo) {
  const int hh = threadIdx.x & 1;
  const int64_t S = (K + 255) / 256;
  const uint8_t* tb = wt + (row >> 4) * S * 2304;
  const int n = (int)(row & 15);
  src.wc = tb + 1024 * hh + 16 * n;
  src.ws = tb + 2048 + 4 * n + 2 * hh;
  src.k_lo = k_lo;
}

__device__ __forceinline__ void gemm_zero_acc(f32x16 (&acc)[kXBlocks][kWBlocks]) {
#pragma unroll
  for (int i = 0; i < kXBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kWBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// The whole K loop of one tile for a wave with XL live activation blocks;
// dma_live: the wave's 32-row band of the activation copy is needed.
// late(src) completes the sources after the first weight loads are issued and
// before the first activation copy (gathered rows: the weight loads then
// overlap the wait for the row indices).
template <bool A_FQ, int XL, bool TW, typename Late>
__device__ __forceinline__ void gemm_mainloop_xl(f32x16 (&acc)[kXBlocks][kWBlocks], char* lds,
                                                 GemmSrc& src, const uint8_t* a_tile_base,
                                                 int64_t K, bool dma_live, Late late) {
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int steps = (int)((K + BK - 1) / BK);
  const int steps2 = (steps + 1) & ~1;  // the loop runs step pairs; a padding step adds zeros
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
    if constexpr (!A_FQ)
      if (dma_live)
        dma_a_tile(lds + buf * kTileBytes, src, a_tile_base, kstep(s), kstep(s) + BK <= K);
  };

  GemmLoad<A_FQ> L0, L1;
  Frags f[2];
  gemm_load<A_FQ, TW>(L0, src, a_tile_base, K, kstep(0));
  gemm_load<A_FQ, TW>(L1, src, a_tile_base, K, kstep(1));
  late(src);
  dma(0, 0);
#pragma unroll
  for (int c = 0; c < 8; ++c) gemm_store_piece<A_FQ>(lds, o, 0, L0, c, kval(0));
  lds_barrier<A_FQ ? -1 : 0>();
#pragma unroll
  for (int i = 0; i < kXBlocks; ++i) read_frag<XL>(f[0], lds, o, 0, 0, i);
  // At step s: buffer s&1 holds step s, set L[(s+1)&1] holds step s+1 (loaded
  // during step s-1) and set L[s&1] is free and takes step s+2.  The buffer
  // written during the last step is not read.  The scheduling barriers keep
  // each step's global loads at its start, ahead of their use.
  for (int s = 0; s < steps2; s += 2) {
    dma(s + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load<A_FQ, TW>(L0, src, a_tile_base, K, kstep(s + 2));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_FQ, XL>(acc, f, lds, o, 0, 1, L1, kval(s + 1));
    dma(s + 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load<A_FQ, TW>(L1, src, a_tile_base, K, kstep(s + 3));
    __builtin_amdgcn_sched_barrier(0);
    gemm_step<A_FQ, XL>(acc, f, lds, o, 1, 0, L0, kval(s + 2));
  }
}

// The whole K loop of one tile: acc += a_tile . w_tile^T.  `lds` is the
// kLdsBytes of dynamic LDS; every thread of the workgroup calls it.
// PARTIAL: only tile rows below live_rows are ever stored, so a wave skips the
// MFMAs and operand reads of its 32-row activation blocks past them and a
// wave whose copy band lies past them skips its activation copy (each wave
// runs the loop specialised for its live blocks; all of them still load and
// decode the weight tile and meet at every barrier).
struct NoLateSrc {
  __device__ void operator()(GemmSrc&) const {}
};

template <bool A_FQ, bool PARTIAL = false, bool TW = false, typename Late = NoLateSrc>
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[kXBlocks][kWBlocks], char* lds,
                                              GemmSrc& src, const uint8_t* a_tile_base, int64_t K,
                                              int live_rows = BM, Late late = Late()) {
  if constexpr (PARTIAL) {
    const int wave = threadIdx.x >> 6;
    const int first = (wave >> 1) * 64;  // the wave's first activation row
    const bool dma_live = 32 * wave < live_rows;
    if (live_rows > first + 32)
      gemm_mainloop_xl<A_FQ, 2, TW>(acc, lds, src, a_tile_base, K, dma_live, late);
    else if (live_rows > first)
      gemm_mainloop_xl<A_FQ, 1, TW>(acc, lds, src, a_tile_base, K, dma_live, late);
    else
      gemm_mainloop_xl<A_FQ, 0, TW>(acc, lds, src, a_tile_base, K, dma_live, late);
  } else {
    gemm_mainloop_xl<A_FQ, 2, TW>(acc, lds, src, a_tile_base, K, true, late);
  }
}

// Output coordinates of accumulator register e of acc[i][j] in thread t:
// tile row wm*64 + i*32 + l%32, tile column wn*128 + j*32 + 8*(e/4) +
// 4*(l/32) + e%4 (registers 4q .. 4q+3 are 4 consecutive columns; wave
// t/64 = 2 wm + wn, lane l = t%64).
__device__ __forceinline__ int acc_row(int t, int i) {
  return ((t >> 6) >> 1) * 64 + i * 32 + (t & 31);
}
__device__ __forceinline__ int acc_col(int t, int j, int q) {
  return ((t >> 6) & 1) * 128 + j * 32 + 8 * q + 4 * ((t & 63) >> 5);
}
__device__ __forceinline__ int gemm_tile_row(int i) { return acc_row(threadIdx.x, i); }
__device__ __forceinline__ int gemm_tile_col(int j, int q) { return acc_col(threadIdx.x, j, q); }

// A tile's fp32 partial sums (a shared tile's segment) are kept in register
// order: group g = (i * kWBlocks + j) * 4 + q (4 consecutive columns) of
// thread t at f32x4 index g * kGemmThreads + t, so each store instruction of
// a wave writes 1 KB contiguous (the tile's row-major order put 16 bytes into
// each of 32 rows per instruction: 7.6 us of stores per segment against 2.7).

// Output staging.  An accumulator block's natural store writes 16 bytes into
// each of 32 rows per instruction (32 partly written cache lines); once the K
// loop is done the operand buffers are free, so the bf16 output tile is
// written to LDS as [256 rows][C columns] (16-byte pieces of a row swizzled
// by the row, so the 32 rows of one write land on distinct banks) and stored
// from there a whole row run per 16 lanes (C = 256: 64 lanes cover two rows
// of 512 contiguous bytes).
template <int C>
__device__ __forceinline__ uint32_t stage_off(int row, int col) {
  constexpr int P = C / 8;  // 16-byte pieces per row
  return (uint32_t)(row * (C * 2) + (((col >> 3) ^ (row % P)) << 4) + (col & 7) * 2);
}

// Four consecutive bf16 outputs (packed) at tile (row, col), col % 4 == 0.
template <int C>
__device__ __forceinline__ void stage_put(char* lds, int row, int col, const u32x2& v) {
  lds_ref<u32x2>(lds, stage_off<C>(row, col)) = v;
}

// Store tile rows [0, nrows) x columns [0, ncols) (ncols % 8 == 0) of the
// staged tile; row_ptr(r) is the 16-byte aligned output address of row r's
// first tile column.  Every thread of the workgroup calls it, after a
// barrier that follows the last stage_put.
template <int C, typename RowPtr>
__device__ __forceinline__ void stage_store(char* lds, int nrows, int ncols, RowPtr row_ptr) {
  constexpr int P = C / 8, kRowsPerPass = kGemmThreads / P;
  const int t = threadIdx.x, p = t % P;
  if (8 * p >= ncols) return;
  for (int r = t / P; r < nrows; r += kRowsPerPass)
    *reinterpret_cast<u32x4*>(row_ptr(r) + 8 * p) =
        lds_ref<const u32x4>(lds, (uint32_t)(r * (C * 2)) + ((p ^ (r % P)) << 4));
}

}  // namespace nvfp4
