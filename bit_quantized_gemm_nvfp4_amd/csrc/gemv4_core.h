// gemv4_core.h -- weight-streaming inner loop for very small M (M <= 8) built on
// the 16-block 4x4x4 bf16 MFMA (internal).
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4x4x4 products; lane l
// belongs to block b = l / 4 and supplies A_b[l % 4][k0..3] and
// B_b[k0..3][l % 4]; C_b[r][l % 4] lands in accumulator register r of lane l.
//
// Lane (b = lane / 4, n = lane % 4) of a wave owns the 32 contiguous elements
// [32b, 32b+32) of weight row n in each 512-element step: one 16-byte code
// load (a wave reads 4 rows x 256 contiguous bytes) and one 2-byte scale load
// (4 rows x 32 contiguous bytes).  Its 32 elements are two NVFP4 blocks of 16
// with one E4M3 scale each, so the scale is applied once per block to the
// MFMA result instead of to every weight:
//     C_tmp = sum of 4 MFMAs over the block's 16 elements (unscaled e2m1 in bf16)
//     acc  += scale * C_tmp
// The e2m1 codes are decoded exactly to bf16 by the hardware converter (scale
// operand 1.0).  A_b rows are activation rows 4*g + (lane % 4), g = the m-group.
// The 16 blocks of the MFMA hold 16 different K pieces of the same 4 weight
// rows; they are summed across lanes once at the end (gemv4_reduce).
#pragma once

#include "device.h"
#include "gemv_core.h"

namespace nvfp4 {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

constexpr int kG4Step = 512;  // K elements per step (16 lanes x 32)

__device__ __forceinline__ f32x4 mfma_4x4x4_bf16(uint32_t a01, uint32_t a23, uint32_t b01,
                                                 uint32_t b23, f32x4 c) {
  const u32x2 av = {a01, a23}, bv = {b01, b23};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, av),
                                                __builtin_bit_cast(s16x4, bv), c, 0, 0, 0);
}

template <int TR>
struct G4Step {
  u32x4 c[TR];       // 32 elements of the lane's row, low nibble first
  uint32_t sc[TR];   // the two E4M3 scales of those elements (bytes 0, 1)
};

template <int TR, bool TAIL>
__device__ __forceinline__ void g4_load(G4Step<TR>& b, const uint8_t* const (&cptr)[TR],
                                        const uint8_t* const (&sptr)[TR], int64_t K, int s) {
  const int blk = (threadIdx.x & 63) >> 2;
  const int64_t k0 = (int64_t)s * kG4Step + 32 * blk;
  const bool ok = !TAIL || k0 + 32 <= K;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const u32x4* cp = reinterpret_cast<const u32x4*>(cptr[t] + k0 / 2);
    b.c[t] = ok ? __builtin_nontemporal_load(cp) : z;
    b.sc[t] = ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(sptr[t] + k0 / 16) : 0u;
  }
}

// One step.  xl[g]: this lane's activation row of m-group g in LDS, at the
// lane's first element of the step.
template <int MG, int TR>
__device__ __forceinline__ void g4_compute(f32x4 (&acc)[TR][MG], const G4Step<TR>& b,
                                           const uint16_t* const (&xl)[MG]) {
  u32x4 a[MG][4];  // 32 activations per m-group: words 2j, 2j+1 feed MFMA j
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) a[g][i] = *reinterpret_cast<const u32x4*>(xl[g] + 8 * i);
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const float s0 = e4m3_to_f32<0>(b.sc[t]);
    const float s1 = e4m3_to_f32<1>(b.sc[t]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the lane's two blocks of 16 elements
      f32x4 ct[MG];
#pragma unroll
      for (int g = 0; g < MG; ++g) ct[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // 4 elements = 2 code bytes per MFMA
        const uint32_t w = b.c[t][2 * h + (j >> 1)];
        const uint32_t b01 = __builtin_bit_cast(uint32_t, (j & 1) ? e2m1x2_to_bf16<2>(w)
                                                                   : e2m1x2_to_bf16<0>(w));
        const uint32_t b23 = __builtin_bit_cast(uint32_t, (j & 1) ? e2m1x2_to_bf16<3>(w)
                                                                   : e2m1x2_to_bf16<1>(w));
        const int e = 16 * h + 4 * j;  // element offset within the lane's 32
#pragma unroll
        for (int g = 0; g < MG; ++g) {
          const u32x4& av = a[g][e >> 3];
          const int wi = (e & 7) >> 1;  // word of av holding elements e, e+1
          ct[g] = mfma_4x4x4_bf16(av[wi], av[wi + 1], b01, b23, ct[g]);
        }
      }
      const float sc = h ? s1 : s0;
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][g][r] += sc * ct[g][r];
    }
  }
}

// Steps [s0, s1); steps_full complete 512-element steps, step steps_full (if
// < s1) partial.  Same unconditional-prefetch double buffer as gemv_core.h.
// `stage` is called after the first weight loads are issued (so their latency
// overlaps the activation staging) and before any activation is read.
template <int MG, int TR, typename Stage>
__device__ __forceinline__ void g4_accumulate(f32x4 (&acc)[TR][MG],
                                              const uint8_t* const (&cptr)[TR],
                                              const uint8_t* const (&sptr)[TR],
                                              const uint16_t* const (&xl0)[MG], int64_t K,
                                              int s0, int s1, int steps_full, Stage stage) {
  const int e = s1 < steps_full ? s1 : steps_full;
  int s = s0;
  const uint16_t* xl[MG];
#pragma unroll
  for (int g = 0; g < MG; ++g) xl[g] = xl0[g];
  if (s >= e) stage();
  if (s < e) {
    G4Step<TR> b0, b1;
    g4_load<TR, false>(b0, cptr, sptr, K, s);
    stage();
    while (true) {
      g4_load<TR, false>(b1, cptr, sptr, K, min(s + 1, e - 1));
      __builtin_amdgcn_sched_barrier(0);
      g4_compute<MG, TR>(acc, b0, xl);
#pragma unroll
      for (int g = 0; g < MG; ++g) xl[g] += kG4Step;
      if (++s >= e) break;
      g4_load<TR, false>(b0, cptr, sptr, K, min(s + 1, e - 1));
      __builtin_amdgcn_sched_barrier(0);
      g4_compute<MG, TR>(acc, b1, xl);
#pragma unroll
      for (int g = 0; g < MG; ++g) xl[g] += kG4Step;
      if (++s >= e) break;
    }
  }
  if (s == steps_full && s < s1) {
    G4Step<TR> bt;
    g4_load<TR, true>(bt, cptr, sptr, K, steps_full);
    g4_compute<MG, TR>(acc, bt, xl);
  }
}

// ---- tiled weights ----------------------------------------------------------------
// With tiled weights (tile.hip) a wave streams whole 16-row tiles, and lane l
// takes the same 64 elements as the 16x16 GEMV's lane: row l % 16 of the
// tile, elements [64 q, 64 q + 64) of each 256-element step, q = l / 16
// (WStep, load_wstep_tiled).  The 4x4x4 blocks are assigned accordingly:
// block b = l / 4 holds rows 4 (b % 4) .. + 3 of the tile (one per lane) and
// the quarter q = b / 4, which all four of its lanes share, so an MFMA's four
// k-slots are the same four elements for the block's A rows (activation rows
// 4 g + l % 4, read from LDS) and B columns.  Lane l accumulates C[4 g + r][row
// l % 16] over its quarter; the four quarters are summed across lanes at the
// end (gemv4t_reduce).

// One tiled step (16 MFMAs per m-group and tile: 4 blocks of 16 elements x 4
// k-slots).  xl[g]: this lane's activation row of m-group g in LDS at element
// 64 q of the step.
template <int MG, int TR>
__device__ __forceinline__ void g4t_compute(f32x4 (&acc)[TR][MG], const WStep<TR>& b,
                                            const uint16_t* const (&xl)[MG]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // the lane's block of 16 elements (scale byte j)
    u32x4 a[MG][2];  // 16 activations per m-group: words 2u, 2u+1 feed MFMA u
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      a[g][0] = *reinterpret_cast<const u32x4*>(xl[g] + 16 * j);
      a[g][1] = *reinterpret_cast<const u32x4*>(xl[g] + 16 * j + 8);
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      f32x4 ct[MG];
#pragma unroll
      for (int g = 0; g < MG; ++g) ct[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // 4 elements = 2 code bytes per MFMA
        const uint32_t w = b.c[t][j >> 1][2 * (j & 1) + (u >> 1)];
        const uint32_t b01 = __builtin_bit_cast(uint32_t, (u & 1) ? e2m1x2_to_bf16<2>(w)
                                                                   : e2m1x2_to_bf16<0>(w));
        const uint32_t b23 = __builtin_bit_cast(uint32_t, (u & 1) ? e2m1x2_to_bf16<3>(w)
                                                                   : e2m1x2_to_bf16<1>(w));
#pragma unroll
        for (int g = 0; g < MG; ++g) {
          const u32x4& av = a[g][u >> 1];
          const int wi = 2 * (u & 1);  // words of av holding the MFMA's four elements
          ct[g] = mfma_4x4x4_bf16(av[wi], av[wi + 1], b01, b23, ct[g]);
        }
      }
      float sc;
      switch (j) {
        case 0: sc = e4m3_to_f32<0>(b.sc[t]); break;
        case 1: sc = e4m3_to_f32<1>(b.sc[t]); break;
        case 2: sc = e4m3_to_f32<2>(b.sc[t]); break;
        default: sc = e4m3_to_f32<3>(b.sc[t]); break;
      }
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][g][r] += sc * ct[g][r];
    }
  }
}

// Steps [s0, s1) of tiled weights, all whole; the same unconditional-prefetch
// double buffer as g4_accumulate.  `stage` is called after the first weight
// loads are issued and before any activation is read.
template <int MG, int TR, typename Stage>
__device__ __forceinline__ void g4t_accumulate(f32x4 (&acc)[TR][MG],
                                               const uint8_t* const (&cptr)[TR],
                                               const uint8_t* const (&sptr)[TR],
                                               const uint16_t* const (&xl0)[MG], int s0, int s1,
                                               Stage stage) {
  int s = s0;
  const uint16_t* xl[MG];
#pragma unroll
  for (int g = 0; g < MG; ++g) xl[g] = xl0[g];
  if (s >= s1) {
    stage();
    return;
  }
  WStep<TR> b0, b1;
  load_wstep_tiled<TR, true>(b0, cptr, sptr, s);
  stage();
  while (true) {
    load_wstep_tiled<TR, true>(b1, cptr, sptr, min(s + 1, s1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    g4t_compute<MG, TR>(acc, b0, xl);
#pragma unroll
    for (int g = 0; g < MG; ++g) xl[g] += kGemvStep;
    if (++s >= s1) break;
    load_wstep_tiled<TR, true>(b0, cptr, sptr, min(s + 1, s1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    g4t_compute<MG, TR>(acc, b1, xl);
#pragma unroll
    for (int g = 0; g < MG; ++g) xl[g] += kGemvStep;
    if (++s >= s1) break;
  }
}

// Sum v over the four lanes of one tile row (the quarters q = lane / 16), in
// a fixed order; every lane ends with the total.
__device__ __forceinline__ float gemv4t_reduce(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Sum v over the 16 lanes that share lane % 4 (the 16 MFMA blocks), in a fixed
// butterfly order; every lane ends with the total.
__device__ __forceinline__ float gemv4_reduce(float v) {
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace nvfp4
