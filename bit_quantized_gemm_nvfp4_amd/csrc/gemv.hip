// gemv.hip -- decode-shaped NVFP4 linear layer (small M) for gfx950.
//
// y[m][j] = sum_k x[m][k] * w[n_j][k], w = e2m1(code) * e4m3(scale) (NVFP4:
// "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding head",
// section "What the artifact is"; W4A16: "What 350+ Experiments Taught Us
// About Serving Qwen 3.6 35B-A3B", section 1).  With row_idx only the listed
// weight rows are read ("The masked head trick" on the first page).
//
// The weights are read exactly once, so the kernel is bound by HBM.  Grid:
// blockIdx.x picks nw*TR tiles of 16 weight rows (TR per wave), blockIdx.y a
// contiguous part of K (split-K across workgroups when the rows alone cannot
// fill the chip, or when the activations of all of K do not fit LDS).  Each
// workgroup stages the activations of its K part in LDS; each wave streams its
// own rows over that part (gemv_core.h).  With one K part the wave stores its
// bf16/fp32 results directly; otherwise it stores fp32 partials and
// k_splitk_reduce adds them in part order, so results are bit-identical from
// run to run.
#include "gemv4_core.h"
#include "gemv_core.h"
#include "launch.h"

namespace nvfp4 {

namespace {

struct GemvArgs {
  const uint16_t* x;       // bf16 [M][K]
  const uint8_t* wc;       // codes [N][K/2]
  const uint8_t* ws;       // scales [N][K/16]
  const int32_t* row_idx;  // optional [n_out]
  void* out;               // [M][n_out] bf16 or fp32 (gridDim.y == 1)
  float* partial;          // fp32 [gridDim.y][M][n_out] (gridDim.y > 1)
  int64_t K;
  int64_t n_out;
  int M;
  int steps;               // ceil(K / step) for the kernel's step size
  int out_f32;
  int fq;                  // activations quantized to NVFP4 and dequantized on staging
  const float* ga;         // two-level scales: the output is multiplied by
  const float* gw;         // *ga * *gw (null: 1); applied to final sums only
};

// TL: the weights are tiled (tile.hip; a.wc is the tiled array, a.ws unused)
// and every step is whole.  WR: rows of the activation window, 16, or 8 for
// M <= 8 on tiled weights (half the window's loads, conversions and LDS
// stores; lanes 8..15 read row 7, whose results are never stored).
template <int MT, int TR, int NW, bool FQ, bool TL = false, int WR = 16>
__global__ void __launch_bounds__(64 * NW) k_gemv(GemvArgs a) {
  static_assert(WR == 16 || (WR == 8 && MT == 1 && TL), "8-row window: tiled, one tile");
  // activation pieces per thread and step (with 8 rows and 8 waves, half the
  // threads stage one piece each)
  constexpr int XP = (WR * MT * 32 + 64 * NW - 1) / (64 * NW);
  // Scale blocks and the fp16 path fit the register budget of 4 waves per SIMD
  // with one activation tile, and with two tiles in 16-wave workgroups (one
  // window piece per thread); with two tiles in smaller workgroups they cost a
  // wave per SIMD, more than the fetched bytes and vector instructions they
  // save.
  // Tiled weights bring their scales in the step's own loads: no scale blocks.
  constexpr bool BLK = !TL && (MT == 1 || NW == 16);
  // fp16 path (plain W4A16): steps whose activations are exact in fp16 run
  // the fp16 MFMA on weights decoded with packed fp16 multiplies (half the
  // vector instructions).  The fused W4A4 staging keeps the bf16 path.
  constexpr bool H = !FQ && (MT == 1 || NW == 16);
  __shared__ uint16_t win[2 * WR * MT * kXWin];  // bf16, or fp16 (H)
  __shared__ int hflag[2];
  __shared__ uint32_t scl[BLK ? NW * TR * 512 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15, q = lane >> 4;
  const int64_t K = a.K;

  const int zs0 = (int)(((int64_t)a.steps * blockIdx.y) / gridDim.y);
  const int zs1 = (int)(((int64_t)a.steps * (blockIdx.y + 1)) / gridDim.y);

  const int64_t tile0 = ((int64_t)blockIdx.x * NW + wave) * TR;
  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
  if constexpr (TL) {
    const int64_t last = (a.n_out + 15) / 16 - 1;
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const int64_t tile = min(tile0 + t, last);  // padding tile: never stored
      const uint8_t* tb = a.wc + tile * a.steps * 2304;
      cptr[t] = tb + 16 * lane;
      sptr[t] = tb + 2048 + 4 * lane;
    }
  } else {
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      int64_t j = (tile0 + t) * 16 + ln;
      if (j >= a.n_out) j = a.n_out - 1;  // padding column: any valid row, never stored
      const int64_t row = a.row_idx ? (int64_t)a.row_idx[j] : j;
      cptr[t] = a.wc + row * (K / 2);
      sptr[t] = a.ws + row * (K / 16);
    }
  }
  int xrow_off[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xrow_off[mt] = (WR == 8 ? min(ln, 7) : 16 * mt + ln) * kXWin + 64 * win_quarter(q);

  f32x4 acc[TR][MT];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* x = a.x;
  auto row_ptr = [x, K](int m) { return x + (int64_t)m * K; };
  if constexpr (H) {  // no step is marked inexact yet
    if (threadIdx.x < 2) hflag[threadIdx.x] = -1;
    __syncthreads();
  }
  bool blocks = false;
  if constexpr (BLK) {
    blocks = K % 256 == 0;
    if (blocks)
      gemv_accumulate_win_blk<MT, TR, XP, FQ, H>(acc, cptr, sptr, win, hflag,
                                                 scl + wave * TR * 512, xrow_off, a.M, K,
                                                 zs0, zs1, row_ptr);
  }
  if (!blocks)
    gemv_accumulate_win<MT, TR, XP, FQ, H, TL, WR>(acc, cptr, sptr, win, hflag, xrow_off, a.M,
                                                   K, zs0, zs1,
                                                   TL ? a.steps : (int)(K / kGemvStep), row_ptr);

  // lane holds C[m = 16*mt + 4*q + r][column 16*tile + ln]
  const bool scaled = gridDim.y == 1 && (a.ga || a.gw);
  const float alpha = scaled ? alpha_of(a.ga, a.gw) : 1.0f;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t j = (tile0 + t) * 16 + ln;
    if (j >= a.n_out) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + 4 * q + r;
        if (m >= a.M) continue;
        const int64_t o = (int64_t)m * a.n_out + j;
        const float v = scaled ? acc[t][mt][r] * alpha : acc[t][mt][r];
        if (gridDim.y > 1)
          a.partial[(int64_t)blockIdx.y * a.M * a.n_out + o] = v;
        else if (a.out_f32)
          static_cast<float*>(a.out)[o] = v;
        else
          static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_bits(v);
      }
    }
  }
}

// K parts inside the workgroup (gemv_accumulate_kp): G groups of TR weight
// tiles x KP parts of the workgroup's K steps, summed in LDS in part order,
// so a K range too long for the rows alone to fill the chip needs neither a
// second kernel nor fp32 partials in memory.  Plain W4A16, one or two
// activation tiles, K % 256 == 0.  blockIdx.x picks G*TR tiles, blockIdx.y a
// K range (z > 1: fp32 partials summed by k_splitk_reduce, as k_gemv).
// TL: tiled weights (a.wc; K need not be a multiple of 256).
template <int MT, int TR, int G, int KP, int WR, bool TL = false>
__global__ void __launch_bounds__(64 * G * KP) k_gemv_kp(GemvArgs a) {
  constexpr int NW = G * KP;
  constexpr int RPP = WR * MT;
  constexpr int XP = KP * RPP * 32 / (64 * NW);  // window pieces per thread and step
  static_assert(XP * 64 * NW == KP * RPP * 32, "window pieces must divide the workgroup");
  static_assert((KP - 1) * G * TR * MT * 64 * 16 <= 2 * KP * RPP * kXWin * 2,
                "the parts' sums must fit the window");
  __shared__ __attribute__((aligned(16))) uint16_t win[2 * KP * RPP * kXWin];
  __shared__ int hflag[2 * KP];
  __shared__ uint32_t scl[TL ? 1 : NW * TR * 512];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = wave % G, part = wave / G;
  const int ln = lane & 15, q = lane >> 4;
  const int64_t K = a.K;
  const int zs0 = (int)(((int64_t)a.steps * blockIdx.y) / gridDim.y);
  const int zs1 = (int)(((int64_t)a.steps * (blockIdx.y + 1)) / gridDim.y);

  const int64_t tile0 = ((int64_t)blockIdx.x * G + g) * TR;
  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
  if constexpr (TL) {
    const int64_t last = (a.n_out + 15) / 16 - 1;
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const int64_t tile = min(tile0 + t, last);  // padding tile: never stored
      const uint8_t* tb = a.wc + tile * a.steps * 2304;
      cptr[t] = tb + 16 * lane;
      sptr[t] = tb + 2048 + 4 * lane;
    }
  } else {
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      int64_t j = (tile0 + t) * 16 + ln;
      if (j >= a.n_out) j = a.n_out - 1;  // padding column: any valid row, never stored
      const int64_t row = a.row_idx ? (int64_t)a.row_idx[j] : j;
      cptr[t] = a.wc + row * (K / 2);
      sptr[t] = a.ws + row * (K / 16);
    }
  }
  f32x4 acc[TR][MT];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x < 2 * KP) hflag[threadIdx.x] = -1;  // no step is marked inexact yet
  __syncthreads();
  const uint16_t* x = a.x;
  gemv_accumulate_kp<MT, TR, XP, KP, WR, true, TL>(acc, cptr, sptr, win, hflag,
                                                   scl + (TL ? 0 : wave * TR * 512), part, a.M,
                                                   K, zs0,
                                               zs1 - zs0,
                                               [x, K](int m) { return x + (int64_t)m * K; });
  gemv_kp_reduce<MT, TR, KP>(acc, reinterpret_cast<f32x4*>(win), part, g, G);
  if (part != 0) return;

  // lane holds C[m = 16*mt + 4*q + r][column 16*tile + ln]
  const bool scaled = gridDim.y == 1 && (a.ga || a.gw);
  const float alpha = scaled ? alpha_of(a.ga, a.gw) : 1.0f;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t j = (tile0 + t) * 16 + ln;
    if (j >= a.n_out) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + 4 * q + r;
        if (m >= a.M) continue;
        const int64_t o = (int64_t)m * a.n_out + j;
        const float v = scaled ? acc[t][mt][r] * alpha : acc[t][mt][r];
        if (gridDim.y > 1)
          a.partial[(int64_t)blockIdx.y * a.M * a.n_out + o] = v;
        else if (a.out_f32)
          static_cast<float*>(a.out)[o] = v;
        else
          static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_bits(v);
      }
    }
  }
}

// Very small M (<= 8): 4x4x4-block MFMA with per-block scaling of the MFMA
// result (gemv4_core.h).  blockIdx.x picks nw*TR tiles of 4 weight rows, a wave
// TR of them; blockIdx.y a contiguous part of K.
template <int MG, int TR, bool FQ>
__global__ void __launch_bounds__(512) k_gemv4(GemvArgs a) {
  extern __shared__ uint16_t xs[];  // [M][steps of this part * 512 + kXPad]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int cn = lane & 3, blk = lane >> 2;
  const int64_t K = a.K;

  const int zs0 = (int)(((int64_t)a.steps * blockIdx.y) / gridDim.y);
  const int zs1 = (int)(((int64_t)a.steps * (blockIdx.y + 1)) / gridDim.y);
  const int nsteps = zs1 - zs0;
  const uint16_t* x = a.x;
  const int stride = nsteps * kG4Step + kXPad;
  auto stage = [&]() {
    stage_activations<FQ>(xs, a.M, (int64_t)zs0 * kG4Step, nsteps * kG4Step, stride, K,
                      [x, K](int m) { return x + (int64_t)m * K; });
  };

  const int64_t tile0 = ((int64_t)blockIdx.x * nw + wave) * TR;
  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    int64_t j = (tile0 + t) * 4 + cn;
    if (j >= a.n_out) j = a.n_out - 1;  // padding column: any valid row, never stored
    const int64_t row = a.row_idx ? (int64_t)a.row_idx[j] : j;
    cptr[t] = a.wc + row * (K / 2);
    sptr[t] = a.ws + row * (K / 16);
  }
  const uint16_t* xl[MG];
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    const int m = min(4 * g + cn, a.M - 1);  // padding row: never stored
    xl[g] = xs + m * stride + 32 * blk;
  }

  f32x4 acc[TR][MG];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[t][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  g4_accumulate<MG, TR>(acc, cptr, sptr, xl, K, zs0, zs1, (int)(K / kG4Step), stage);

  // acc[t][g][r] of lane (blk, cn) is block blk's part of row 4g+r, column
  // 4*tile + cn; sum the 16 blocks, then lane blk == m stores row m.
  const bool scaled = gridDim.y == 1 && (a.ga || a.gw);
  const float alpha = scaled ? alpha_of(a.ga, a.gw) : 1.0f;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t j = (tile0 + t) * 4 + cn;
#pragma unroll
    for (int g = 0; g < MG; ++g) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * g + r;
        if (m >= a.M) continue;  // uniform
        const float s4 = gemv4_reduce(acc[t][g][r]);
        const float v = scaled ? s4 * alpha : s4;
        if (blk != m || j >= a.n_out) continue;
        const int64_t o = (int64_t)m * a.n_out + j;
        if (gridDim.y > 1)
          a.partial[(int64_t)blockIdx.y * a.M * a.n_out + o] = v;
        else if (a.out_f32)
          static_cast<float*>(a.out)[o] = v;
        else
          static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_bits(v);
      }
    }
  }
}

// Very small M (<= 8) on tiled weights: the 4x4x4-block MFMA with per-block
// scaling (g4t_compute).  blockIdx.x picks G*TR tiles of 16 weight rows
// (G = waves / KP), blockIdx.y a contiguous range of K steps (256 elements)
// whose activations are staged in LDS.  Wave w streams the TR tiles of group
// w % G over part w / G of that range (KP contiguous parts); the parts' sums
// are added in LDS in part order (gemv_kp_reduce), so a K range too long for
// the rows alone to fill the chip needs no second kernel.
template <int MG, int TR, int KP>
__global__ void __launch_bounds__(KP > 1 ? 1024 : 512) k_gemv4_tiled(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [M][range * 256 + kXPad]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = (blockDim.x >> 6) / KP;  // tile groups
  const int g = wave % nw, part = wave / nw;
  const int ln = lane & 15, q = lane >> 4;
  const int64_t K = a.K;

  const int zs0 = (int)(((int64_t)a.steps * blockIdx.y) / gridDim.y);
  const int zs1 = (int)(((int64_t)a.steps * (blockIdx.y + 1)) / gridDim.y);
  const int nsteps = zs1 - zs0;
  const uint16_t* x = a.x;
  const int stride = nsteps * kTileStep + kXPad;
  auto stage = [&]() {
    stage_activations<false>(xs, a.M, (int64_t)zs0 * kTileStep, nsteps * kTileStep, stride, K,
                             [x, K](int m) { return x + (int64_t)m * K; });
  };

  const int64_t tile0 = ((int64_t)blockIdx.x * nw + g) * TR;
  const int64_t last = (a.n_out + 15) / 16 - 1;
  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t tile = min(tile0 + t, last);  // padding tile: never stored
    const uint8_t* tb = a.wc + tile * a.steps * 2304;
    cptr[t] = tb + 16 * lane;
    sptr[t] = tb + 2048 + 4 * lane;
  }
  const KParts me = kpart(zs0, nsteps, part, KP);
  const uint16_t* xl[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int m = min(4 * mg + (lane & 3), a.M - 1);  // padding row: never stored
    xl[mg] = xs + m * stride + (me.start - zs0) * kTileStep + 64 * q;
  }

  f32x4 acc[TR][MG];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[t][mg] = f32x4{0.f, 0.f, 0.f, 0.f};

  g4t_accumulate<MG, TR>(acc, cptr, sptr, xl, me.start, me.start + me.len, stage);
  if constexpr (KP > 1) {
    __syncthreads();  // every wave is done with the staged activations
    gemv_kp_reduce<MG, TR, KP>(acc, reinterpret_cast<f32x4*>(xs), part, g, nw);
    if (part != 0) return;
  }

  // acc[t][g][r] of lane (q, ln) is quarter q's part of activation row 4g+r,
  // weight row 16*tile + ln; sum the quarters, then lane q == r % 4 stores.
  const bool scaled = gridDim.y == 1 && (a.ga || a.gw);
  const float alpha = scaled ? alpha_of(a.ga, a.gw) : 1.0f;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t j = (tile0 + t) * 16 + ln;
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * mg + r;
        if (m >= a.M) continue;  // uniform
        const float s4 = gemv4t_reduce(acc[t][mg][r]);
        const float v = scaled ? s4 * alpha : s4;
        if (q != r || j >= a.n_out) continue;
        const int64_t o = (int64_t)m * a.n_out + j;
        if (gridDim.y > 1)
          a.partial[(int64_t)blockIdx.y * a.M * a.n_out + o] = v;
        else if (a.out_f32)
          static_cast<float*>(a.out)[o] = v;
        else
          static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_bits(v);
      }
    }
  }
}

// Sum of the K parts of a split-K launch, in part order (bit-identical from
// run to run).  A thread owns V consecutive outputs (V = 4 when count % 4 ==
// 0 and the output is aligned for 4-element stores).  The parts are loaded in
// batches of up to eight whose loads are all in flight before the adds, so the
// sum waits about one memory latency per eight parts instead of one per part.
template <int V>
__device__ __forceinline__ void load_part(float (&d)[V], const float* p) {
  if constexpr (V == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p);
    d[0] = t[0], d[1] = t[1], d[2] = t[2], d[3] = t[3];
  } else {
    d[0] = *p;
  }
}

// v += parts z0 .. z0+B-1 (in that order) at p = partial + i.
template <int B, int V>
__device__ __forceinline__ void add_parts(float (&v)[V], const float* p, int64_t count, int z0) {
  float q[B][V];
#pragma unroll
  for (int j = 0; j < B; ++j) load_part<V>(q[j], p + (int64_t)(z0 + j) * count);
#pragma unroll
  for (int j = 0; j < B; ++j)
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] += q[j][e];
}

template <int V>
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* __restrict__ partial,
                                                       int splits, int64_t count, int out_f32,
                                                       const float* ga, const float* gw,
                                                       void* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (i >= count) return;
  const float* p = partial + i;
  float v[V];
#pragma unroll
  for (int e = 0; e < V; ++e) v[e] = 0.f;
  int z = 0;
  for (; z + 8 <= splits; z += 8) add_parts<8, V>(v, p, count, z);
  switch (splits - z) {  // the last batch (uniform)
    case 1: add_parts<1, V>(v, p, count, z); break;
    case 2: add_parts<2, V>(v, p, count, z); break;
    case 3: add_parts<3, V>(v, p, count, z); break;
    case 4: add_parts<4, V>(v, p, count, z); break;
    case 5: add_parts<5, V>(v, p, count, z); break;
    case 6: add_parts<6, V>(v, p, count, z); break;
    case 7: add_parts<7, V>(v, p, count, z); break;
    default: break;
  }
  if (ga || gw) {
    const float alpha = alpha_of(ga, gw);
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] *= alpha;
  }
  if constexpr (V == 4) {
    if (out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
      const u32x2 pk = {(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                        (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i) = pk;
    }
  } else {
    if (out_f32)
      static_cast<float*>(out)[i] = v[0];
    else
      static_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v[0]);
  }
}

template <int MT, int TR, bool FQ>
void launch_gemv_t(const GemvArgs& a, int nw, int zsplit, hipStream_t stream) {
  const int64_t tiles = (a.n_out + 15) / 16;
  const int64_t per_wg = (int64_t)nw * TR;
  dim3 grid((unsigned)((tiles + per_wg - 1) / per_wg), (unsigned)zsplit);
  if constexpr (MT == 2 && TR <= 2) {
    // 16 waves: plan_gemv asks for them only here (the window has one piece
    // per thread and the kernel fits 128 registers)
    if (nw == 16) {
      hipLaunchKernelGGL((k_gemv<MT, TR, 16, FQ>), grid, dim3(1024), 0, stream, a);
      return;
    }
  }
  if (nw == 8)
    hipLaunchKernelGGL((k_gemv<MT, TR, 8, FQ>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((k_gemv<MT, TR, 4, FQ>), grid, dim3(256), 0, stream, a);
}

// Sum of the z > 1 K parts of a split-K GEMV launch (nothing when z == 1).
int splitk_reduce(int z, int64_t M, int64_t n_out, bool out_f32, void* out, void* workspace,
                  Alpha alpha, hipStream_t stream) {
  if (z <= 1) return 0;
  const int64_t count = M * n_out;
  const float* part = static_cast<const float*>(workspace);
  const uintptr_t oa = reinterpret_cast<uintptr_t>(out) % (out_f32 ? 16 : 8);
  if (count % 4 == 0 && oa == 0)
    hipLaunchKernelGGL(k_splitk_reduce<4>, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256),
                       0, stream, part, z, count, out_f32 ? 1 : 0, alpha.a, alpha.w, out);
  else
    hipLaunchKernelGGL(k_splitk_reduce<1>, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       stream, part, z, count, out_f32 ? 1 : 0, alpha.a, alpha.w, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int MT, int TR, int WR = 16>
int launch_gemv_tiled_t(const GemvArgs& a, int nw, int zsplit, hipStream_t stream) {
  const int64_t tiles = (a.n_out + 15) / 16;
  const int64_t per_wg = (int64_t)nw * TR;
  dim3 grid((unsigned)((tiles + per_wg - 1) / per_wg), (unsigned)zsplit);
  if constexpr (MT == 2) {
    if (nw == 16) {
      hipLaunchKernelGGL((k_gemv<MT, TR, 16, false, true>), grid, dim3(1024), 0, stream, a);
      return 0;
    }
  }
  if (nw == 8)
    hipLaunchKernelGGL((k_gemv<MT, TR, 8, false, true, WR>), grid, dim3(512), 0, stream, a);
  else if (nw == 4)
    hipLaunchKernelGGL((k_gemv<MT, TR, 4, false, true, WR>), grid, dim3(256), 0, stream, a);
  else
    return -2;
  return 0;
}

// The K-parts layouts that are built: (tiles per wave, tile groups, parts).
struct KpLayout {
  int tr, g, kp;
};
constexpr KpLayout kKpLayouts[] = {{2, 2, 4}, {2, 4, 2}, {1, 4, 4}, {2, 2, 8}, {1, 2, 8},
                                   {2, 1, 8}, {1, 4, 2}};

template <int MT, int WR, int TR, int G, int KP, bool TL = false>
bool try_kp(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
  if (p.tr != TR || p.nw != G * KP || p.kp != KP) return false;
  const int64_t tiles = (a.n_out + 15) / 16;
  dim3 grid((unsigned)((tiles + G * TR - 1) / (G * TR)), (unsigned)p.z);
  hipLaunchKernelGGL((k_gemv_kp<MT, TR, G, KP, WR, TL>), grid, dim3(64 * G * KP), 0, stream, a);
  return true;
}

template <int MT, int WR>
int launch_gemv_kp_tl(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
  bool ok = try_kp<MT, WR, 2, 2, 4, true>(a, p, stream) ||
            try_kp<MT, WR, 2, 4, 2, true>(a, p, stream) ||
            try_kp<MT, WR, 1, 4, 4, true>(a, p, stream) ||
            try_kp<MT, WR, 1, 4, 2, true>(a, p, stream);
  if constexpr (WR == 8)
    ok = ok || try_kp<MT, WR, 2, 2, 8, true>(a, p, stream) ||
         try_kp<MT, WR, 1, 2, 8, true>(a, p, stream) || try_kp<MT, WR, 2, 1, 8, true>(a, p, stream);
  return ok ? 0 : -2;
}

template <int MT, int WR>
int launch_gemv_kp_t(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
  bool ok = try_kp<MT, WR, 2, 2, 4>(a, p, stream) || try_kp<MT, WR, 2, 4, 2>(a, p, stream) ||
            try_kp<MT, WR, 1, 4, 4>(a, p, stream) || try_kp<MT, WR, 1, 4, 2>(a, p, stream);
  if constexpr (WR == 8)  // eight parts fit LDS with 8-row windows only
    ok = ok || try_kp<MT, WR, 2, 2, 8>(a, p, stream) || try_kp<MT, WR, 1, 2, 8>(a, p, stream) ||
         try_kp<MT, WR, 2, 1, 8>(a, p, stream);
  return ok ? 0 : -2;
}

template <int MG, int TR, bool FQ>
void launch_gemv4_t(const GemvArgs& a, int nw, int zsplit, hipStream_t stream) {
  const int64_t tiles = (a.n_out + 3) / 4;
  const int64_t per_wg = (int64_t)nw * TR;
  dim3 grid((unsigned)((tiles + per_wg - 1) / per_wg), (unsigned)zsplit);
  const int max_steps = (a.steps + zsplit - 1) / zsplit;
  const size_t lds = (size_t)a.M * (max_steps * kG4Step + kXPad) * sizeof(uint16_t);
  hipLaunchKernelGGL((k_gemv4<MG, TR, FQ>), grid, dim3(64 * nw), lds, stream, a);
}

// The plan's (tiles per wave) choice as a template argument; fused W4A4
// staging is instantiated for the plan's defaults (one or two tiles per wave).
template <bool SMALL, int MT, int TR>
int launch_plan(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
  if (a.fq) {
    if constexpr (TR <= 2) {
      if constexpr (SMALL)
        launch_gemv4_t<MT, TR, true>(a, p.nw, p.z, stream);
      else
        launch_gemv_t<MT, TR, true>(a, p.nw, p.z, stream);
      return 0;
    }
    return -2;
  }
  if constexpr (SMALL)
    launch_gemv4_t<MT, TR, false>(a, p.nw, p.z, stream);
  else
    launch_gemv_t<MT, TR, false>(a, p.nw, p.z, stream);
  return 0;
}

}  // namespace

GemvPlan plan_gemv(int64_t M, int64_t n_out, int64_t K, int num_cus, const PlanOverride& ov,
                   bool tiled) {
  GemvPlan p;
  // largest M for the 4x4x4-block kernel with per-block scaling
  const int64_t small_max = ov.gemv_small_max >= 0 ? ov.gemv_small_max : 4;
  p.small = M <= small_max;
  p.mt = p.small ? (int)((M + 3) / 4) : (M <= 16 ? 1 : 2);
  // tiled weights: the 4x4x4 kernel's tiles are 16 rows, one per wave
  p.tr = tiled && p.small ? 1 : 2;
  // Wide workgroups (8 waves; on the 16x16 path they share one activation
  // window) when there are rows enough to fill the chip with them, 4 waves
  // otherwise (measured: the 248,320-row head at M = 1 takes ~10% less time
  // with 8 waves, the 17,408-row layers are as fast or faster with 4).  With
  // two activation tiles, 16 waves (scale blocks and the fp16 path; one
  // workgroup per CU, 99 KB of LDS with two weight tiles per wave, 66 KB with
  // one): two tiles per wave once they give at least 256 workgroups, one
  // below (measured at M = 32 against 8 and 4 waves: the 248,320-row head
  // 204 -> 177 us, the 32,768-row masked head 38 -> 33 us, the 17,408-row
  // layers 33-34 -> 28-29 us).
  p.nw = n_out >= 32768 ? 8 : 4;
  if (!p.small && p.mt == 2) {
    p.nw = 16;
    p.tr = n_out >= 256 * 512 ? 2 : 1;
  }
  // overrides (tuning entry points): tiles per wave, waves per workgroup, the
  // LDS budget of the staged activations, the number of K parts
  if (ov.gemv_tiles >= 0) p.tr = ov.gemv_tiles;
  if (ov.gemv_waves >= 0) p.nw = ov.gemv_waves;
  const int64_t lds_budget = ov.gemv_lds_kib >= 0 ? (int64_t)ov.gemv_lds_kib * 1024 : 64 * 1024;
  const int64_t step = p.small && !tiled ? kG4Step : kGemvStep;
  const int64_t rows_per_tile = p.small && !tiled ? 4 : 16;
  const int64_t steps = (K + step - 1) / step;
  int64_t z = 1;
  if (p.small) {  // the 4x4x4 kernel stages its whole K part: it must fit LDS
    int64_t max_steps = (lds_budget / (2 * M) - kXPad) / step;
    if (max_steps < 1) max_steps = 1;
    z = (steps + max_steps - 1) / max_steps;
  }
  const int64_t z_lds = z;
  // enough waves to fill the chip
  const int64_t tiles = (n_out + rows_per_tile - 1) / rows_per_tile;
  const int64_t wgs = (tiles + (int64_t)p.nw * p.tr - 1) / ((int64_t)p.nw * p.tr);
  if (p.nw == 16) {
    // one workgroup per CU (LDS, registers): as many K parts as keep every
    // workgroup in one round (measured at M = 32: the 17,408 x 5,120 layer
    // 44 / 36 / 28 us with 4 / 6 / 9 parts, the masked head 48 -> 35 us with
    // 2 parts instead of 1, a second round costing more than it splits)
    const int64_t zc = num_cus / wgs;
    if (zc > z) z = zc;
  } else {
    const int64_t want_waves = (int64_t)num_cus * 8;
    int64_t zw = (want_waves + wgs * p.nw - 1) / (wgs * p.nw);
    // a layer that needs K parts to fill the chip takes parts of at most 4
    // steps on the 16x16 path: a workgroup's steps run one after another, each
    // about one memory latency (measured at M = 8: the 17,408 x 5,120 layer
    // 21.5 -> 19.4 us with 5 parts instead of 4, the 5,120 x 17,408 layer
    // 22.4 -> 19.5 us with 17 instead of 13)
    if (!p.small && zw >= 2 && (steps + 3) / 4 > zw) zw = (steps + 3) / 4;
    if (zw > z) z = zw;
  }
  if (ov.gemv_splits > 0) z = ov.gemv_splits > z_lds ? ov.gemv_splits : z_lds;
  if (z > steps) z = steps;
  if (z < 1) z = 1;
  p.z = (int)z;
  // K parts inside the workgroup (override only, for now): the workgroup's
  // waves are tile groups x parts
  p.kp = 1;
  // K parts inside the workgroup instead of across workgroups, for M <= 8 on
  // layers wide enough for 1.5 workgroups of 4 tiles per CU (measured at M = 8:
  // the 32,768-row masked head 27.7 -> 23.8 us; on the 17,408-row layer the
  // 272 workgroups leave some CUs with two and the split-K launch is as fast)
  // (the same on tiled weights: the 32,768-row masked head at M = 8 25.9 ->
  // 19.3 us graph-replayed)
  const bool kp_default = ov.gemv_kparts < 0 && ov.gemv_tiles < 0 && ov.gemv_waves < 0 &&
                          ov.gemv_splits < 0 && !p.small && M <= 8 &&
                          (tiled || K % kGemvStep == 0) &&
                          p.z >= 2 && steps >= 2 && (tiles + 3) / 4 >= (int64_t)num_cus * 3 / 2;
  if (kp_default) {
    p.tr = 1;
    p.nw = 8;
    p.kp = 2;
    p.z = 1;
  }
  // Tiled weights, 4x4x4 kernel, layers of fewer than 8 tiles per CU: K parts
  // inside the workgroup instead of across workgroups (no reduce launch), two
  // tile groups per workgroup, enough parts for about 2,048 waves (measured at
  // M = 1, graph-replayed: the 17,408 x 5,120 layer 13.0 -> 11.5 us with 2
  // parts, the 5,120 x 17,408 layer 13.2 -> 12.0 us with 8)
  if (tiled && p.small && ov.gemv_kparts < 0 && ov.gemv_tiles < 0 && ov.gemv_waves < 0 &&
      ov.gemv_splits < 0 && tiles < (int64_t)num_cus * 8) {
    int64_t kp = 2;
    while (kp < 8 && tiles * kp < 2048) kp *= 2;
    while (kp > 1 && kp * z_lds > steps) kp /= 2;
    if (kp > 1) {
      p.kp = (int)kp;
      p.tr = 1;
      p.nw = 2 * (int)kp;
      p.z = (int)z_lds;
    }
  }
  if (ov.gemv_kparts > 1 && (tiled || (!p.small && K % kGemvStep == 0))) {
    p.kp = ov.gemv_kparts;
    if (ov.gemv_splits <= 0) p.z = z_lds;
    if ((int64_t)p.z * p.kp > steps) p.z = (int)(steps / p.kp);  // every part >= 1 step
    if (p.z < 1) p.z = 1;
  }
  return p;
}

bool gemv_override_valid(int64_t M, int64_t K, const PlanOverride& ov) {
  if (ov.gemv_small_max > 8) return false;
  if (ov.gemv_lds_kib >= 0 && (ov.gemv_lds_kib < 8 || ov.gemv_lds_kib > 160)) return false;
  const GemvPlan p = plan_gemv(M, 1, K, kNumCUs, ov);
  if (ov.gemv_kparts > 1) {  // a built K-parts layout: full steps, one activation tile
                             // (two: 1 tile per wave, 16 waves, 2 parts)
    if (p.small || K % kGemvStep != 0 || K / kGemvStep < ov.gemv_kparts) return false;
    if (p.mt == 2) return p.tr == 1 && p.nw == 16 && ov.gemv_kparts == 2;
    if (ov.gemv_kparts == 8 && M > 8) return false;  // 16-row windows: at most 4 parts
    for (const KpLayout& l : kKpLayouts)
      if (l.tr == p.tr && l.g * l.kp == p.nw && l.kp == ov.gemv_kparts) return true;
    return false;
  }
  const bool tr_ok = p.small ? (p.tr == 1 || p.tr == 2 || p.tr == 4 || (p.tr == 8 && p.mt == 1))
                             : (p.tr == 1 || p.tr == 2 || (p.tr == 4 && p.mt == 1));
  const bool nw_ok = p.small ? (p.nw >= 1 && p.nw <= 8)
                             : (p.nw == 4 || p.nw == 8 || (p.nw == 16 && p.mt == 2 && p.tr <= 2));
  return tr_ok && nw_ok;
}

size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t n_out) {
  return p.z > 1 ? (size_t)p.z * (size_t)M * (size_t)n_out * sizeof(float) : 0;
}

int launch_gemv(const GemvPlan& p, const uint16_t* x, int64_t M, int64_t K, const uint8_t* wc,
                const uint8_t* ws, const int32_t* row_idx, int64_t n_out, bool out_f32,
                void* out, void* workspace, hipStream_t stream, Alpha alpha,
                bool fakequant) {
  GemvArgs a;
  a.fq = fakequant ? 1 : 0;
  a.ga = alpha.a;
  a.gw = alpha.w;
  a.x = x;
  a.wc = wc;
  a.ws = ws;
  a.row_idx = row_idx;
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.K = K;
  a.n_out = n_out;
  a.M = (int)M;
  const int64_t step = p.small ? kG4Step : kGemvStep;
  a.steps = (int)((K + step - 1) / step);
  a.out_f32 = out_f32 ? 1 : 0;
  int rc = -2;
  if (p.kp > 1 && !fakequant) {
    if (p.mt == 1 && M <= 8)
      rc = launch_gemv_kp_t<1, 8>(a, p, stream);
    else if (p.mt == 1)
      rc = launch_gemv_kp_t<1, 16>(a, p, stream);
    else if (p.mt == 2 && try_kp<2, 16, 1, 8, 2>(a, p, stream))
      rc = 0;
  } else if (p.small) {
    if (p.mt == 1 && p.tr == 4)
      rc = launch_plan<true, 1, 4>(a, p, stream);
    else if (p.mt == 1 && p.tr == 2)
      rc = launch_plan<true, 1, 2>(a, p, stream);
    else if (p.mt == 1 && p.tr == 8)
      rc = launch_plan<true, 1, 8>(a, p, stream);
    else if (p.mt == 1 && p.tr == 1)
      rc = launch_plan<true, 1, 1>(a, p, stream);
    else if (p.mt == 2 && p.tr == 4)
      rc = launch_plan<true, 2, 4>(a, p, stream);
    else if (p.mt == 2 && p.tr == 2)
      rc = launch_plan<true, 2, 2>(a, p, stream);
    else if (p.mt == 2 && p.tr == 1)
      rc = launch_plan<true, 2, 1>(a, p, stream);
  } else if (p.mt == 1 && p.tr == 2)
    rc = launch_plan<false, 1, 2>(a, p, stream);
  else if (p.mt == 1 && p.tr == 1)
    rc = launch_plan<false, 1, 1>(a, p, stream);
  else if (p.mt == 1 && p.tr == 4)
    rc = launch_plan<false, 1, 4>(a, p, stream);
  else if (p.mt == 2 && p.tr == 2)
    rc = launch_plan<false, 2, 2>(a, p, stream);
  else if (p.mt == 2 && p.tr == 1)
    rc = launch_plan<false, 2, 1>(a, p, stream);
  if (rc != 0) return rc;
  if (hipGetLastError() != hipSuccess) return -1;
  return splitk_reduce(p.z, M, n_out, out_f32, out, workspace, alpha, stream);
}

// nw waves = tile groups x kp parts.
template <int MG, int TR, int KP>
int launch_gemv4_tiled_t(const GemvArgs& a, int nw, int zsplit, hipStream_t stream) {
  const int64_t tiles = (a.n_out + 15) / 16;
  const int64_t per_wg = (int64_t)(nw / KP) * TR;
  dim3 grid((unsigned)((tiles + per_wg - 1) / per_wg), (unsigned)zsplit);
  const int max_steps = (a.steps + zsplit - 1) / zsplit;
  const size_t stage = (size_t)a.M * (max_steps * kTileStep + kXPad) * sizeof(uint16_t);
  const size_t red = (size_t)(KP - 1) * (nw / KP) * TR * MG * 64 * 16;
  hipLaunchKernelGGL((k_gemv4_tiled<MG, TR, KP>), grid, dim3(64 * nw),
                     stage > red ? stage : red, stream, a);
  return 0;
}

int launch_gemv_tiled(const GemvPlan& p, const uint16_t* x, int64_t M, int64_t K,
                      const uint8_t* wt, int64_t N, bool out_f32, void* out, void* workspace,
                      hipStream_t stream, Alpha alpha) {
  GemvArgs a;
  a.fq = 0;
  a.ga = alpha.a;
  a.gw = alpha.w;
  a.x = x;
  a.wc = wt;
  a.ws = nullptr;
  a.row_idx = nullptr;
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.K = K;
  a.n_out = N;
  a.M = (int)M;
  a.steps = (int)((K + kTileStep - 1) / kTileStep);
  a.out_f32 = out_f32 ? 1 : 0;
  int rc = -2;
  if (p.small) {
    if (p.mt == 1 && p.tr == 1 && p.kp == 1)
      rc = launch_gemv4_tiled_t<1, 1, 1>(a, p.nw, p.z, stream);
    else if (p.mt == 1 && p.tr == 2 && p.kp == 1)
      rc = launch_gemv4_tiled_t<1, 2, 1>(a, p.nw, p.z, stream);
    else if (p.mt == 2 && p.tr == 1 && p.kp == 1)
      rc = launch_gemv4_tiled_t<2, 1, 1>(a, p.nw, p.z, stream);
    else if (p.mt == 1 && p.tr == 1 && p.kp == 2)
      rc = launch_gemv4_tiled_t<1, 1, 2>(a, p.nw, p.z, stream);
    else if (p.mt == 1 && p.tr == 1 && p.kp == 4)
      rc = launch_gemv4_tiled_t<1, 1, 4>(a, p.nw, p.z, stream);
    else if (p.mt == 1 && p.tr == 1 && p.kp == 8)
      rc = launch_gemv4_tiled_t<1, 1, 8>(a, p.nw, p.z, stream);
    else if (p.mt == 1 && p.tr == 1 && p.kp == 16)
      rc = launch_gemv4_tiled_t<1, 1, 16>(a, p.nw, p.z, stream);
  } else if (p.kp > 1) {
    if (p.mt == 1 && a.M <= 8)
      rc = launch_gemv_kp_tl<1, 8>(a, p, stream);
    else if (p.mt == 1)
      rc = launch_gemv_kp_tl<1, 16>(a, p, stream);
    else if (p.mt == 2 && try_kp<2, 16, 1, 8, 2, true>(a, p, stream))
      rc = 0;
  } else if (p.mt == 1 && M <= 8) {  // 8-row window (measured, graph-replayed at M = 8:
    // 16.2 -> 15.7 us on the 17,408 x 5,120 layer, 115.4 -> 113.1 us on the 248,320-row head)
    if (p.tr == 2)
      rc = launch_gemv_tiled_t<1, 2, 8>(a, p.nw, p.z, stream);
    else if (p.tr == 1)
      rc = launch_gemv_tiled_t<1, 1, 8>(a, p.nw, p.z, stream);
    else if (p.tr == 4)
      rc = launch_gemv_tiled_t<1, 4, 8>(a, p.nw, p.z, stream);
  } else if (p.mt == 1 && p.tr == 2)
    rc = launch_gemv_tiled_t<1, 2>(a, p.nw, p.z, stream);
  else if (p.mt == 1 && p.tr == 1)
    rc = launch_gemv_tiled_t<1, 1>(a, p.nw, p.z, stream);
  else if (p.mt == 1 && p.tr == 4)
    rc = launch_gemv_tiled_t<1, 4>(a, p.nw, p.z, stream);
  else if (p.mt == 2 && p.tr == 2)
    rc = launch_gemv_tiled_t<2, 2>(a, p.nw, p.z, stream);
  else if (p.mt == 2 && p.tr == 1)
    rc = launch_gemv_tiled_t<2, 1>(a, p.nw, p.z, stream);
  if (rc != 0) return rc;
  if (hipGetLastError() != hipSuccess) return -1;
  return splitk_reduce(p.z, M, N, out_f32, out, workspace, alpha, stream);
}

}  // namespace nvfp4
