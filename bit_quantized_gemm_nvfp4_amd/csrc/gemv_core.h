// gemv_core.h -- the weight-streaming inner loop shared by the decode GEMV and
// the grouped (mixture-of-experts) GEMV kernels (internal).
//
// A workgroup stages the activations of its K range in LDS once (coalesced
// 16-byte loads), then each wave streams the NVFP4 codes and scales of its own
// TR tiles of 16 weight rows over that K range, 256 elements per step, and
// accumulates with bf16 MFMA.  Keeping the activations out of the per-step
// vector-memory loads leaves the texture-address path to the weights alone.
//
// Lane (n = lane % 16, q = lane / 16) owns, per step and weight tile, the 64
// contiguous elements [64q, 64q+64) of weight row n: two 16-byte code words and
// the four scale bytes that cover them (one 32-bit load).  A wave's code loads
// cover 16 rows x 128 contiguous bytes.  Each 32-bit code word (8 elements, one
// scale) is decoded exactly to bf16 in registers and is the B operand of one
// v_mfma_f32_16x16x32_bf16 (B[k][n]: lane holds k-slots 8*(lane/16) .. +7 of
// column lane%16).  The A operand (read from LDS) carries the matching 8
// activations of activation row lane % 16, so an MFMA's 32 k-slots map to
// scattered physical k; any bijection gives the same dot product as long as A
// and B agree.
//
// With one activation tile (M <= 16), and with two in 16-wave workgroups, the
// plain W4A16 GEMV runs most steps in fp16 instead: the window holds the
// activations converted to fp16, checked to be exact, and the codes are
// decoded to fp16 with one packed fp16 multiply per pair (e2m1 * E4M3 has <= 6
// significant bits inside fp16's normal range), for v_mfma_f32_16x16x32_f16.  Every product is the same exact value as on
// the bf16 path, with half the vector instructions per weight; a step whose
// activations are not all exact in fp16 runs the bf16 path.
//
// Code/scale loads of step s+1 are issued before step s is computed (register
// double buffer, pinned with scheduling barriers).  Main-loop loads are
// unconditional: weight rows past the end are clamped to a valid row and
// activation rows past M read a valid row -- both only feed accumulator
// entries that are never stored.  Only the last step, when K is not a multiple
// of 256, takes the masked path (K % 32 == 0: each 32-element half of a lane's
// range is either in or out); its absent elements get zero codes, zero scales
// and zero-filled activations.
//
// Result layout: lane holds C[m = 4*(lane/16) + r][n = lane % 16], r = 0..3.
#pragma once

#include <type_traits>

#include "device.h"
#include "quant_core.h"

namespace nvfp4 {

constexpr int kGemvStep = 256;  // K elements per step
constexpr int kXPad = 8;        // bf16 elements of padding per LDS activation row

template <int TR>
struct WStep {
  u32x4 c[TR][2];   // code words: elements [64q, 64q+32) and [64q+32, 64q+64)
  uint32_t sc[TR];  // the four E4M3 scale bytes of those 64 elements
};

// LDS row stride (bf16 elements) for a K range of `steps` 256-element steps.
__host__ __device__ inline int lds_x_stride(int steps) { return steps * kGemvStep + kXPad; }

// Stage activation rows [0, m_rows) x [k_lo, k_lo + klen) into LDS as
// [m_rows][stride] bf16; elements at or past K are zero.  row_ptr(m) gives the
// global row (bf16, K elements).  klen % 8 == 0.  All threads of the workgroup
// take part; ends with a barrier.
//
// FQ (W4A4 with bf16 activations): every 16-element block is quantized to
// NVFP4 and dequantized on the way (fakequant_piece; a block's two pieces are
// neighbouring lanes), so the GEMM sees exactly the activations a separate
// nvfp4_quantize + nvfp4_dequantize would give.
template <bool FQ = false, typename RowPtr>
__device__ __forceinline__ void stage_activations(uint16_t* lds, int m_rows, int64_t k_lo,
                                                  int klen, int stride, int64_t K,
                                                  RowPtr row_ptr) {
  const int chunks_per_row = klen / 8;
  const int total = m_rows * chunks_per_row;
  const u32x4 z = {0u, 0u, 0u, 0u};
  // Four pieces per thread are loaded before any is stored, so the staging
  // waits about one memory latency per four rounds instead of one per round.
  // (total and blockDim.x are even, so a block's two lanes are active together)
  for (int c0 = threadIdx.x; c0 < total; c0 += 4 * blockDim.x) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * blockDim.x;
      const int m = c / chunks_per_row, c8 = c - m * chunks_per_row;
      const int64_t k = k_lo + (int64_t)c8 * 8;
      v[u] = (c < total && k < K) ? *reinterpret_cast<const u32x4*>(row_ptr(m) + k) : z;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * blockDim.x;
      if (c >= total) break;
      const int m = c / chunks_per_row, c8 = c - m * chunks_per_row;
      u32x4 w = v[u];
      if constexpr (FQ) w = fakequant_piece(w);
      *reinterpret_cast<u32x4*>(lds + m * stride + c8 * 8) = w;
    }
  }
  __syncthreads();
}

template <int TR, bool TAIL>
__device__ __forceinline__ void load_wstep(WStep<TR>& b, const uint8_t* const (&cptr)[TR],
                                           const uint8_t* const (&sptr)[TR], int64_t K,
                                           bool scale_dword, int s) {
  const int q = (threadIdx.x & 63) >> 4;
  const int64_t k0 = (int64_t)s * kGemvStep + 64 * q;  // first element of this lane
  const bool h0 = !TAIL || k0 + 32 <= K;                // halves present (tail step only)
  const bool h1 = !TAIL || k0 + 64 <= K;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const uint8_t* c = cptr[t] + k0 / 2;
    const uint8_t* sc = sptr[t] + k0 / 16;
    if (TAIL) {
      b.c[t][0] = h0 ? *reinterpret_cast<const u32x4*>(c) : z;
      b.c[t][1] = h1 ? *reinterpret_cast<const u32x4*>(c + 16) : z;
      const uint32_t lo = h0 ? *reinterpret_cast<const uint16_t*>(sc) : 0u;
      const uint32_t hi = h1 ? *reinterpret_cast<const uint16_t*>(sc + 2) : 0u;
      b.sc[t] = lo | (hi << 16);
    } else {
      b.c[t][0] = *reinterpret_cast<const u32x4*>(c);
      b.c[t][1] = *reinterpret_cast<const u32x4*>(c + 16);
      if (scale_dword)
        b.sc[t] = *reinterpret_cast<const uint32_t*>(sc);
      else
        b.sc[t] = (uint32_t)*reinterpret_cast<const uint16_t*>(sc) |
                  ((uint32_t)*reinterpret_cast<const uint16_t*>(sc + 2) << 16);
    }
  }
}

// Tiled weights (tile.hip): cptr[t] = the wave's tile block 0 + 16 * lane,
// sptr[t] = the tile's block 0 + 2048 + 4 * lane; step s is block s of the
// tile (2,304 bytes further per step).  The lane gets the same 64 elements
// and four scale bytes as load_wstep's lane (n, q), read as three contiguous
// runs per wave.  Every step is whole (the layout pads K with zero codes and
// scales).
// NT: non-temporal code loads.
template <int TR, bool NT = false>
__device__ __forceinline__ void load_wstep_tiled(WStep<TR>& b, const uint8_t* const (&cptr)[TR],
                                                 const uint8_t* const (&sptr)[TR], int s) {
  const int64_t o = (int64_t)s * 2304;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const u32x4* c = reinterpret_cast<const u32x4*>(cptr[t] + o);
    if constexpr (NT) {
      b.c[t][0] = __builtin_nontemporal_load(c);
      b.c[t][1] = __builtin_nontemporal_load(c + 64);
    } else {
      b.c[t][0] = c[0];
      b.c[t][1] = c[64];
    }
    b.sc[t] = *reinterpret_cast<const uint32_t*>(sptr[t] + o);
  }
}

// A whole step from either layout.  Tiled codes are loaded non-temporally
// (streamed past the caches; measured at M = 8: the 248,320 x 5,120 head
// 129 -> 116 us), row-major codes are not (their scale blocks and the
// 16-byte pieces of one line arrive in separate requests).
template <int TR, bool TL>
__device__ __forceinline__ void load_wstep_full(WStep<TR>& b, const uint8_t* const (&cptr)[TR],
                                                const uint8_t* const (&sptr)[TR], int64_t K,
                                                bool scale_dword, int s) {
  if constexpr (TL)
    load_wstep_tiled<TR, true>(b, cptr, sptr, s);
  else
    load_wstep<TR, false>(b, cptr, sptr, K, scale_dword, s);
}

// One step: A operands from LDS (xl[mt]: this lane's activation row in LDS at
// the step's element 64q), B operands decoded from the codes.  The A operands
// are read one 8-element chunk at a time, one chunk ahead of their MFMAs, so
// only two chunks per m-tile are live (fewer registers, more waves per SIMD).
// H: the A operands are fp16 (the fp16 window copy) and the weights are
// decoded to fp16 with packed multiplies (dequant8_f16) for the fp16 MFMA;
// every product is the same exact value as on the bf16 path.
template <int MT, int TR, bool H = false>
__device__ __forceinline__ void compute_wstep(f32x4 (&acc)[TR][MT], const WStep<TR>& b,
                                              const uint16_t* const (&xl)[MT]) {
  auto ld = [&](int mt, int j) { return *reinterpret_cast<const u32x4*>(xl[mt] + 8 * j); };
  float s[TR][4];
  f16x2 sh[TR][2];  // fp16 scales of blocks (0, 1) and (2, 3)
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    if constexpr (H) {
      sh[t][0] = e4m3x2_to_f16<false>(b.sc[t]);
      sh[t][1] = e4m3x2_to_f16<true>(b.sc[t]);
    } else {
      s[t][0] = e4m3_to_f32<0>(b.sc[t]);
      s[t][1] = e4m3_to_f32<1>(b.sc[t]);
      s[t][2] = e4m3_to_f32<2>(b.sc[t]);
      s[t][3] = e4m3_to_f32<3>(b.sc[t]);
    }
  }
  u32x4 a[2][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) a[0][mt] = ld(mt, 0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j + 1 < 8) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[(j + 1) & 1][mt] = ld(mt, j + 1);
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      if constexpr (H) {
        const f16x2 sp = sh[t][j >> 2];
        const u32x4 w = dequant8_f16(b.c[t][j >> 2][j & 3], ((j >> 1) & 1) ? sp.y : sp.x);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = mfma_16x16x32_f16(a[j & 1][mt], w, acc[t][mt]);
      } else {
        const u32x4 w = dequant8_bf16(b.c[t][j >> 2][j & 3], s[t][j >> 1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = mfma_16x16x32_bf16(a[j & 1][mt], w, acc[t][mt]);
      }
    }
  }
}

// Accumulate steps [s0, s1) (absolute step indices).  xl0[mt] points at this
// lane's activation row in LDS at element 64q of step s0.  `steps_full` is the
// number of complete 256-element steps of K; step steps_full (if < s1) is the
// partial last step.
// TL: tiled weights (load_wstep_tiled pointers), every step whole.
template <int MT, int TR, bool TL = false>
__device__ __forceinline__ void gemv_accumulate(f32x4 (&acc)[TR][MT],
                                                const uint8_t* const (&cptr)[TR],
                                                const uint8_t* const (&sptr)[TR],
                                                const uint16_t* const (&xl0)[MT], int64_t K,
                                                int s0, int s1, int steps_full) {
  const bool sdw = (K % 64) == 0;  // scale rows 4-byte aligned
  const int e = s1 < steps_full ? s1 : steps_full;  // end of the unmasked steps
  int s = s0;
  const uint16_t* xl[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xl[mt] = xl0[mt];
  if (s < e) {
    // Prefetches are unconditional so the compiler can count outstanding loads
    // exactly; past the last step they re-read it and the data is unused.  The
    // scheduling barriers keep each prefetch batch ahead of the compute it
    // overlaps.
    WStep<TR> b0, b1;
    load_wstep_full<TR, TL>(b0, cptr, sptr, K, sdw, s);
    while (true) {
      load_wstep_full<TR, TL>(b1, cptr, sptr, K, sdw, min(s + 1, e - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute_wstep<MT, TR>(acc, b0, xl);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xl[mt] += kGemvStep;
      if (++s >= e) break;
      load_wstep_full<TR, TL>(b0, cptr, sptr, K, sdw, min(s + 1, e - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute_wstep<MT, TR>(acc, b1, xl);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xl[mt] += kGemvStep;
      if (++s >= e) break;
    }
  }
  if (!TL && s == steps_full && s < s1) {  // partial last step
    WStep<TR> bt;
    load_wstep<TR, true>(bt, cptr, sptr, K, sdw, steps_full);
    compute_wstep<MT, TR>(acc, bt, xl);
  }
}

// Activation window: the workgroup streams the activations through a double
// buffer of two 256-element steps in LDS ([2][16*MT][kXWin] bf16), one step
// ahead of the weights, with one barrier per step.  The window always holds
// 16*MT rows (rows past M repeat row M-1) so every thread moves the same
// number of 16-byte pieces, XP = 16*MT*32 / blockDim, with no branches: loads
// past K read a clamped address and are replaced by zero.
constexpr int kXWin = kGemvStep + kXPad;  // LDS row stride of the window

// Inside a window row the 64-element quarters 1 and 2 trade places.  gfx950
// serves a 16-byte LDS read 32 lanes at a time over 512 bytes of banks; the
// operand reads of lanes (n, q) and (n, q + 1) fall on rows n and n' with
// chunks 16 n and 16 n' + 128 modulo 512 bytes (rows 528 bytes apart), which
// collide for n = n' + 8.  With the swap the two quarters of a 32-lane group
// sit 256 bytes apart and all 32 chunks differ (measured with
// SQ_LDS_BANK_CONFLICT: 4 conflict cycles per read -> 0).
__host__ __device__ constexpr int win_quarter(int q) { return ((q & 1) << 1) | (q >> 1); }
// Element offset, inside a window row, of its 8-element chunk cc (0..31).
__device__ __forceinline__ int win_chunk(int cc) {
  return 64 * win_quarter(cc >> 3) + 8 * (cc & 7);
}

// WR: window rows (16, or 8 for M <= 8 with one activation tile: 256 pieces,
// threads past them idle).
template <int XP, int WR = 16, typename RowPtr>
__device__ __forceinline__ void xwin_load(u32x4 (&v)[XP], int M, int64_t K, int s,
                                          RowPtr row_ptr) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (WR < 16 && c >= WR * 32) continue;
    const int m = min(c >> 5, M - 1), c8 = c & 31;
    const int64_t k = (int64_t)s * kGemvStep + c8 * 8;
    const u32x4 t = *reinterpret_cast<const u32x4*>(row_ptr(m) + min(k, K - 8));
    v[i] = k < K ? t : z;
  }
}

// Fused W4A4 activations: quantize and dequantize the loaded pieces in place
// (piece c and c ^ 1 of a window row form one block; they are neighbouring
// lanes).  Done just before the pieces are stored, so the loads stay in flight
// over the step's compute.
template <bool FQ, int XP>
__device__ __forceinline__ void xwin_fakequant(u32x4 (&v)[XP]) {
  if constexpr (FQ) {
#pragma unroll
    for (int i = 0; i < XP; ++i) v[i] = fakequant_piece(v[i]);
  }
}

template <int XP, int WR = 16>
__device__ __forceinline__ void xwin_store(uint16_t* buf, const u32x4 (&v)[XP]) {
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (WR < 16 && c >= WR * 32) continue;
    *reinterpret_cast<u32x4*>(buf + (c >> 5) * kXWin + win_chunk(c & 31)) = v[i];
  }
}

// fp16 window (H): the window holds the steps' activations converted to fp16,
// and a step whose activations are not all exact in fp16 is marked in the
// workgroup's flag word of its buffer (`hflag[buffer]` = that step's index; a
// stale index of an earlier step never matches, and the kernel sets both words
// to -1 before the first step).  Every inexact lane writes the same value, so
// concurrent LDS writes agree.  The flag is read after the barrier that
// publishes the step; a marked step is staged again in bf16.  Only values
// beyond fp16's range (|x| > 65504) or too small to keep bf16's 8 significant
// bits as fp16 subnormals (|x| < 2^-17) fail: for N(0,1) activations about 1%
// of the steps at M = 8.
//
// A workgroup whose activations fail twice stops converting (`hw.on` false)
// and streams the rest of its K range in bf16, so data full of such values
// costs at most two restaged steps per workgroup.
struct HWin {
  int* flag;  // [2] flag words of the two buffers
  int fails;  // steps restaged so far (workgroup-uniform)
  bool on;    // the window is being filled in fp16
};

template <bool H, int XP, int WR = 16>
__device__ __forceinline__ void xwin_store2(uint16_t* buf, const HWin& hw, int bufidx,
                                            const u32x4 (&v)[XP], int s) {
  if constexpr (H) {
    if (hw.on) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < XP; ++i) {
        const int c = threadIdx.x + i * blockDim.x;
        if (WR < 16 && c >= WR * 32) continue;
        u32x4 h;
        ok = bf16x8_to_f16(v[i], h) && ok;
        *reinterpret_cast<u32x4*>(buf + (c >> 5) * kXWin + win_chunk(c & 31)) = h;
      }
      if (!ok) hw.flag[bufidx] = s;
      return;
    }
  }
  xwin_store<XP, WR>(buf, v);
}

// Before step s is computed from window buffer `buf` (H): true when the
// buffer holds the step in fp16 and its activations are exact there;
// otherwise (marked step) the step is reloaded and stored in bf16 over the
// same buffer, with a barrier (the flag is workgroup-uniform, so every wave
// takes this branch together), and false.  `xv` is free at this point (the next
// step's prefetch is issued after).
template <bool H, int XP, int WR = 16, typename RowPtr>
__device__ __forceinline__ bool xwin_fp16_or_restage(uint16_t* buf, HWin& hw, int bufidx,
                                                     u32x4 (&xv)[XP], int M, int64_t K, int s,
                                                     RowPtr row_ptr) {
  if constexpr (H) {
    if (!hw.on) return false;
    if (__builtin_amdgcn_readfirstlane(hw.flag[bufidx]) != s) return true;
    xwin_load<XP, WR>(xv, M, K, s, row_ptr);
    xwin_store<XP, WR>(buf, xv);
    __syncthreads();
    hw.on = ++hw.fails < 2;
  }
  return false;
}

// One step from window buffer `cur`: fp16 MFMA path or bf16 path.
template <int MT, int TR, int WR = 16>
__device__ __forceinline__ void compute_wstep_win(f32x4 (&acc)[TR][MT], const WStep<TR>& b,
                                                  const uint16_t* win, int cur, bool f16,
                                                  const int (&xrow_off)[MT]) {
  constexpr int wsz = WR * MT * kXWin;
  const uint16_t* xl[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xl[mt] = win + cur * wsz + xrow_off[mt];
  if (f16)
    compute_wstep<MT, TR, true>(acc, b, xl);
  else
    compute_wstep<MT, TR, false>(acc, b, xl);
}

// Accumulate steps [s0, s1) with the activations streamed through the LDS
// window `win` ([2][WR*MT][kXWin]; bf16, or fp16 with `hflag` when H).
// xrow_off[mt] = (16*mt + lane%16) * kXWin + 64 * win_quarter(q) (rows past M hold copies,
// their results are never stored); with 8 window rows (WR = 8, MT = 1, M <= 8)
// lanes 8..15 read row 7 (min(lane%16, 7)).  Every thread of the workgroup
// calls this with the same arguments except the weight pointers.  blockDim.x *
// XP >= WR*MT*32 (equal when WR = 16).
template <int MT, int TR, int XP, bool FQ = false, bool H = false, bool TL = false,
          int WR = 16, typename RowPtr>
__device__ __forceinline__ void gemv_accumulate_win(f32x4 (&acc)[TR][MT],
                                                    const uint8_t* const (&cptr)[TR],
                                                    const uint8_t* const (&sptr)[TR],
                                                    uint16_t* win, int* hflag,
                                                    const int (&xrow_off)[MT], int M, int64_t K,
                                                    int s0, int s1, int steps_full,
                                                    RowPtr row_ptr) {
  if (s0 >= s1) return;
  const bool sdw = (K % 64) == 0;  // scale rows 4-byte aligned
  constexpr int wsz = WR * MT * kXWin;
  const int e = s1 < steps_full ? s1 : steps_full;  // end of the full steps
  int s = s0, cur = 0;
  // The first step's weights are requested before the activations are staged,
  // so the two memory latencies overlap instead of adding up.
  WStep<TR> b0, b1;
  if (s < e) load_wstep_full<TR, TL>(b0, cptr, sptr, K, sdw, s);
  u32x4 xv[XP];
  xwin_load<XP, WR>(xv, M, K, s0, row_ptr);
  xwin_fakequant<FQ, XP>(xv);
  HWin hw{hflag, 0, true};
  xwin_store2<H, XP, WR>(win, hw, 0, xv, s0);
  __syncthreads();
  // One step: prefetch the activations of step s+1 and the weights of step
  // s+1 (unconditional: past the end they re-read a valid step and the data
  // is unused), compute step s, publish the activations of step s+1.
  auto stage = [&](WStep<TR>& bc, WStep<TR>& bn) {
    const bool f16 =
        xwin_fp16_or_restage<H, XP, WR>(win + cur * wsz, hw, cur, xv, M, K, s, row_ptr);
    xwin_load<XP, WR>(xv, M, K, min(s + 1, s1 - 1), row_ptr);
    load_wstep_full<TR, TL>(bn, cptr, sptr, K, sdw, min(s + 1, e - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute_wstep_win<MT, TR, WR>(acc, bc, win, cur, f16, xrow_off);
    xwin_fakequant<FQ, XP>(xv);
    xwin_store2<H, XP, WR>(win + (cur ^ 1) * wsz, hw, cur ^ 1, xv, s + 1);
    __syncthreads();
    cur ^= 1;
    return ++s >= e;
  };
  if (s < e) {
    while (true) {
      if (stage(b0, b1)) break;
      if (stage(b1, b0)) break;
    }
  }
  if (!TL && s == steps_full && s < s1) {  // partial last step; its activations are in `cur`
    WStep<TR> bt;
    load_wstep<TR, true>(bt, cptr, sptr, K, sdw, steps_full);
    const bool f16 =
        xwin_fp16_or_restage<H, XP, WR>(win + cur * wsz, hw, cur, xv, M, K, s, row_ptr);
    compute_wstep_win<MT, TR, WR>(acc, bt, win, cur, f16, xrow_off);
  }
}

// ---- scale blocks ---------------------------------------------------------------
// A wave reads its rows' scales 8 steps at a time instead of 4 bytes per lane
// and step: each row's 128 scale bytes of a block are read in two bursts (the
// block's last two steps prefetch the next block, one half each) and kept in
// the wave's own LDS area [TR][8 steps][64 words], word n*4 + q of step j being
// the four scale bytes lane (n, q) uses at that step.  Per-step 16-byte reads
// let the streaming code lines evict a row's scale line between its uses (the
// fetched bytes grew by up to a fifth); block reads fetch each line once.  The
// wave alone writes and reads its area, and LDS operations of one wave
// complete in order, so no barrier is needed.  Rows' scale bytes must be
// 16-byte aligned (K % 256 == 0).

template <int TR>
__device__ __forceinline__ void load_wcodes(WStep<TR>& b, const uint8_t* const (&cptr)[TR], int s) {
  const int q = (threadIdx.x & 63) >> 4;
  const int64_t k0 = (int64_t)s * kGemvStep + 64 * q;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    b.c[t][0] = *reinterpret_cast<const u32x4*>(cptr[t] + k0 / 2);
    b.c[t][1] = *reinterpret_cast<const u32x4*>(cptr[t] + k0 / 2 + 16);
  }
}

// 8-step scale blocks, loaded in two halves: half h of the block starting at
// step B is, for lane (n, q), the 16-byte group of step B + 2q + h of row n;
// it is stored to LDS rows 2q + h ([TR][8 steps][64 words: n*4 + q']).
template <int TR>
__device__ __forceinline__ void load_shalf(u32x4 (&p)[TR], const uint8_t* const (&sptr)[TR], int b,
                                           int h, int last) {
  const int q = (threadIdx.x & 63) >> 4;
  const int st = min(b + 2 * q + h, last);
#pragma unroll
  for (int t = 0; t < TR; ++t) p[t] = *reinterpret_cast<const u32x4*>(sptr[t] + 16 * st);
}

template <int TR>
__device__ __forceinline__ void store_shalf(uint32_t* lds, const u32x4 (&p)[TR], int h) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int t = 0; t < TR; ++t)
    *reinterpret_cast<u32x4*>(lds + t * 512 + (2 * q + h) * 64 + n * 4) = p[t];
}

template <int TR>
__device__ __forceinline__ void read_sblock(WStep<TR>& b, const uint32_t* lds, int j) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int t = 0; t < TR; ++t) b.sc[t] = lds[t * 512 + j * 64 + n * 4 + q];
}

template <int MT, int TR, int XP, bool FQ = false, bool H = false, typename RowPtr>
__device__ __forceinline__ void gemv_accumulate_win_blk(f32x4 (&acc)[TR][MT],
                                                        const uint8_t* const (&cptr)[TR],
                                                        const uint8_t* const (&sptr)[TR],
                                                        uint16_t* win, int* hflag, uint32_t* my,
                                                        const int (&xrow_off)[MT], int M,
                                                        int64_t K, int s0, int s1,
                                                        RowPtr row_ptr) {
  if (s0 >= s1) return;
  constexpr int wsz = 16 * MT * kXWin;
  const int e = s1;  // K % 256 == 0: every step is full
  // The first step's codes and the first scale block are requested before the
  // activations are staged, so their memory latencies overlap.
  WStep<TR> b0, b1;
  load_wcodes<TR>(b0, cptr, s0);
  u32x4 ph[TR], ph1[TR];
  load_shalf<TR>(ph, sptr, s0, 0, e - 1);
  load_shalf<TR>(ph1, sptr, s0, 1, e - 1);
  u32x4 xv[XP];
  xwin_load<XP>(xv, M, K, s0, row_ptr);
  store_shalf<TR>(my, ph, 0);
  store_shalf<TR>(my, ph1, 1);
  xwin_fakequant<FQ, XP>(xv);
  HWin hw{hflag, 0, true};
  xwin_store2<H, XP>(win, hw, 0, xv, s0);
  __syncthreads();
  int s = s0, cur = 0, j = 0;  // j: position of step s in its 8-step block
  auto stage = [&](WStep<TR>& bc, WStep<TR>& bn) {
    const bool f16 = xwin_fp16_or_restage<H, XP>(win + cur * wsz, hw, cur, xv, M, K, s, row_ptr);
    // the next block starts at step s + 8 - j; its two halves are loaded at
    // the block's last two steps, ahead of the window and code prefetches, so
    // the scale store below waits for the scale and window loads only and the
    // codes of step s + 1 stay in flight over the barrier
    const bool sh = j >= 6;
    if (sh) load_shalf<TR>(ph, sptr, s + 8 - j, j - 6, e - 1);
    xwin_load<XP>(xv, M, K, min(s + 1, s1 - 1), row_ptr);
    load_wcodes<TR>(bn, cptr, min(s + 1, e - 1));
    __builtin_amdgcn_sched_barrier(0);
    read_sblock<TR>(bc, my, j);
    compute_wstep_win<MT, TR>(acc, bc, win, cur, f16, xrow_off);
    xwin_fakequant<FQ, XP>(xv);
    xwin_store2<H, XP>(win + (cur ^ 1) * wsz, hw, cur ^ 1, xv, s + 1);
    // half 0 fills rows 0, 2, 4, 6 (row 7 is still read at the last step);
    // half 1 fills rows 1, 3, 5, 7 after it
    if (sh) store_shalf<TR>(my, ph, j - 6);
    __syncthreads();
    cur ^= 1;
    j = (j + 1) & 7;
    return ++s >= e;
  };
  while (true) {
    if (stage(b0, b1)) break;
    if (stage(b1, b0)) break;
  }
}

// ---- K parts inside the workgroup -------------------------------------------------
// A workgroup of G x KP waves: G groups of TR weight tiles, and KP contiguous
// parts of the workgroup's K steps; wave w streams the tiles of group w % G over
// part w / G.  At iteration i every part p processes its step start_p + i, so
// the activation window holds one step per part ([2][KP][WR*MT][kXWin]) and the
// workgroup still meets once per iteration.  The parts' sums are added in LDS
// at the end, in part order (gemv_kp_reduce), so no second kernel and no fp32
// partials in memory are needed.  WR is the number of window rows per
// activation tile: 8 when M <= 8 (rows 8..15 of the MFMA operand read row 7),
// else 16.  Full 256-element steps only (K % 256 == 0), scale blocks, fp16
// path as gemv_accumulate_win_blk.

struct KParts {
  int start;  // first step of the wave's part
  int len;    // its steps (>= 1)
};

__device__ __forceinline__ KParts kpart(int s0, int S, int p, int KP) {
  const int a = (S * p) / KP, b = (S * (p + 1)) / KP;
  return KParts{s0 + a, b - a};
}

// Window pieces of iteration i: piece c of the buffer is row (c >> 5) % (WR*MT)
// of part (c >> 5) / (WR*MT), 8 elements at (c & 31) * 8 of that part's step
// (clamped to the part's last step); rows past M repeat row M-1.
// KCHK: elements at or past K (the last step of tiled weights) read a clamped
// address and are replaced by zero.
template <int XP, int KP, int RPP, bool KCHK = false, typename RowPtr>
__device__ __forceinline__ void xwin_load_kp(u32x4 (&v)[XP], int M, int64_t K, int s0, int S,
                                             int i, RowPtr row_ptr) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int c = threadIdx.x + u * blockDim.x;
    const int p = (c >> 5) / RPP, r = (c >> 5) - p * RPP;
    const KParts kp = kpart(s0, S, p, KP);
    const int s = kp.start + min(i, kp.len - 1);
    const int m = min(r, M - 1);
    const int64_t k = (int64_t)s * kGemvStep + (c & 31) * 8;
    if constexpr (KCHK) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(row_ptr(m) + min(k, K - 8));
      v[u] = k < K ? t : z;
    } else {
      v[u] = *reinterpret_cast<const u32x4*>(row_ptr(m) + k);
    }
  }
}

// Stores the pieces (fp16 when hw.on, marking a part whose values are not all
// exact in fp16 with tag `i` in hflag[buffer][part]; bf16 otherwise).
template <bool H, int XP, int RPP>
__device__ __forceinline__ void xwin_store_kp(uint16_t* buf, int* hflag_buf, bool on,
                                              const u32x4 (&v)[XP], int tag) {
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int c = threadIdx.x + u * blockDim.x;
    uint16_t* dst = buf + (c >> 5) * kXWin + win_chunk(c & 31);
    if (H && on) {
      u32x4 h;
      if (!bf16x8_to_f16(v[u], h)) hflag_buf[(c >> 5) / RPP] = tag;
      *reinterpret_cast<u32x4*>(dst) = h;
    } else {
      *reinterpret_cast<u32x4*>(dst) = v[u];
    }
  }
}

// TL: tiled weights (load_wstep_tiled: codes and scales of a step in one
// set of loads, no scale blocks; K need not be a multiple of 256).
template <int MT, int TR, int XP, int KP, int WR, bool H, bool TL = false, typename RowPtr>
__device__ __forceinline__ void gemv_accumulate_kp(f32x4 (&acc)[TR][MT],
                                                   const uint8_t* const (&cptr)[TR],
                                                   const uint8_t* const (&sptr)[TR],
                                                   uint16_t* win, int* hflag, uint32_t* my,
                                                   int part, int M, int64_t K, int s0, int S,
                                                   RowPtr row_ptr) {
  constexpr int RPP = WR * MT;              // window rows per part
  constexpr int psz = RPP * kXWin;          // one part's rows
  constexpr int wsz = KP * psz;             // one buffer
  const int lane = threadIdx.x & 63, ln = lane & 15, q = lane >> 4;
  const KParts me = kpart(s0, S, part, KP);
  int xrow_off[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xrow_off[mt] =
        part * psz + (WR == 8 ? min(ln, 7) : 16 * mt + ln) * kXWin + 64 * win_quarter(q);
  const int L = (S + KP - 1) / KP;          // iterations (the longest part)
  const int last = me.start + me.len - 1;
  WStep<TR> b0, b1;
  u32x4 ph[TR], ph1[TR];
  if constexpr (TL) {
    load_wstep_tiled<TR, true>(b0, cptr, sptr, me.start);
  } else {
    load_wcodes<TR>(b0, cptr, me.start);
    load_shalf<TR>(ph, sptr, me.start, 0, last);
    load_shalf<TR>(ph1, sptr, me.start, 1, last);
  }
  u32x4 xv[XP];
  xwin_load_kp<XP, KP, RPP, TL>(xv, M, K, s0, S, 0, row_ptr);
  if constexpr (!TL) {
    store_shalf<TR>(my, ph, 0);
    store_shalf<TR>(my, ph1, 1);
  }
  bool on = true;
  int fails = 0;
  xwin_store_kp<H, XP, RPP>(win, hflag, on, xv, 0);
  __syncthreads();
  int i = 0, cur = 0;
  auto stage = [&](WStep<TR>& bc, WStep<TR>& bn) {
    // fp16 unless a part of this buffer was marked at tag i: then the whole
    // buffer is staged again in bf16 (workgroup-uniform, with a barrier)
    bool f16 = false;
    if (H && on) {
      bool marked = false;
#pragma unroll
      for (int p = 0; p < KP; ++p)
        marked = marked || __builtin_amdgcn_readfirstlane(hflag[cur * KP + p]) == i;
      f16 = !marked;
      if (marked) {
        xwin_load_kp<XP, KP, RPP, TL>(xv, M, K, s0, S, i, row_ptr);
        xwin_store_kp<false, XP, RPP>(win + cur * wsz, nullptr, false, xv, 0);
        __syncthreads();
        on = ++fails < 2;
      }
    }
    const int j = i & 7;
    const bool sh = !TL && j >= 6;  // scale halves first, as in gemv_accumulate_win_blk
    if (sh) load_shalf<TR>(ph, sptr, me.start + i + 8 - j, j - 6, last);
    xwin_load_kp<XP, KP, RPP, TL>(xv, M, K, s0, S, min(i + 1, L - 1), row_ptr);
    if constexpr (TL)
      load_wstep_tiled<TR, true>(bn, cptr, sptr, min(me.start + i + 1, last));
    else
      load_wcodes<TR>(bn, cptr, min(me.start + i + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    if (i < me.len) {
      if constexpr (!TL) read_sblock<TR>(bc, my, j);
      const uint16_t* xl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xl[mt] = win + cur * wsz + xrow_off[mt];
      if (f16)
        compute_wstep<MT, TR, true>(acc, bc, xl);
      else
        compute_wstep<MT, TR, false>(acc, bc, xl);
    }
    xwin_store_kp<H, XP, RPP>(win + (cur ^ 1) * wsz, hflag + (cur ^ 1) * KP, on, xv, i + 1);
    if (sh) store_shalf<TR>(my, ph, j - 6);
    __syncthreads();
    cur ^= 1;
    return ++i >= L;
  };
  while (true) {
    if (stage(b0, b1)) break;
    if (stage(b1, b0)) break;
  }
}

// Sum of the KP parts' accumulators in part order, through LDS `red` (every
// wave of the workgroup calls it after the last barrier of the main loop).
// On return the waves of part 0 hold the sums; the other waves' values are
// undefined.  red holds (KP - 1) * G * TR * MT * 64 f32x4.
template <int MT, int TR, int KP>
__device__ __forceinline__ void gemv_kp_reduce(f32x4 (&acc)[TR][MT], f32x4* red, int part, int g,
                                               int G) {
  const int lane = threadIdx.x & 63;
  auto slot = [&](int p, int t, int mt) { return (((p - 1) * G + g) * TR + t) * MT + mt; };
  if (part > 0) {
#pragma unroll
    for (int t = 0; t < TR; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[slot(part, t, mt) * 64 + lane] = acc[t][mt];
  }
  __syncthreads();
  if (part == 0) {
    for (int p = 1; p < KP; ++p) {
#pragma unroll
      for (int t = 0; t < TR; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 v = red[slot(p, t, mt) * 64 + lane];
          acc[t][mt][0] += v[0], acc[t][mt][1] += v[1], acc[t][mt][2] += v[2],
              acc[t][mt][3] += v[3];
        }
    }
  }
}

}  // namespace nvfp4
