// gemm.hip -- prefill-shaped NVFP4 linear layer (large M) for gfx950.
//
// y = a . W^T with W = e2m1(code) * e4m3(scale) (NVFP4: "Serving Qwen3.8-27B in
// 4-bit with a masked speculative decoding head", section "What the artifact
// is"), bf16 activations (W4A16: "What 350+ Experiments Taught Us About Serving
// Qwen 3.6 35B-A3B", section 1) or bf16 activations quantized to NVFP4 as the
// tiles load them (W4A4: "52.6% more tokens, 1.53x less GPU time: production
// inference with Minima and Rafay"), fp32 accumulation.  At M in the thousands
// every weight is reused M times, so the kernel is bound by the bf16 MFMA rate,
// not by HBM.  The 256 x 256 tile is gemm_core.h.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so each XCD is given a contiguous band of the tile sequence, which runs
// over n fastest within groups of 8 m-tiles; the tiles an XCD holds at once
// share activation rows and weight columns in its L2.
#include <algorithm>

#include "gemm_core.h"
#include "launch.h"

namespace nvfp4 {

constexpr int kMaxGemmSegs = 8;  // partial slots per shared tile at most
constexpr int kMinSegSteps = 8;  // K steps per workgroup of a shared round at least

namespace {

struct GemmArgs {
  const uint16_t* a;        // bf16 [M][K]
  const uint8_t* wc;        // weight codes [rows][K/2], or the tiled weights (tiled)
  const uint8_t* ws;        // weight scales [rows][K/16] (row-major only)
  const int32_t* row_idx;   // output column n uses weight row row_idx[n]; null: row n
  void* out;                // [M][N] bf16 or fp32
  float* partial;           // shared tiles: fp32 [tail][max_seg][256 * 256], tile-local
  int64_t M, N, K;          // N: output columns
  int out_f32;
  int tiles_m, tiles_n;
  int full;                 // tiles 0 .. full-1 of the tile order run whole (full % 8 == 0;
                            // workgroups past the last tile exit)
  int tail;                 // tiles full .. full+tail-1 are shared by `parts` workgroups
  int parts;
  int max_seg;
  int steps;                // K steps of 64 (the last may be partial)
  const float* ga;          // two-level scales: final sums are multiplied by
  const float* gw;          // *ga * *gw (null: 1)
};

// The shared round: flattened step f = tail tile * steps + K step, F of them;
// workgroup w takes [w F / P, (w + 1) F / P).  The workgroup holding step f:
__host__ __device__ inline int sk_owner(int64_t f, int64_t F, int P) {
  return (int)(((f + 1) * P - 1) / F);
}

// Tile `lin` of the launch order -> (tm, tn): n fastest within groups of 8
// m-tiles, so the tiles one XCD holds at once share activation rows and
// weight columns in its L2.
__device__ __forceinline__ void gemm_tile_of(int lin, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int group = lin / (GM * tiles_n);
  const int gm0 = group * GM;
  const int gsz = min(GM, tiles_m - gm0);
  const int in_group = lin - group * GM * tiles_n;
  tm = gm0 + in_group % gsz;
  tn = in_group / gsz;
}

// Tile `lin` over K steps [s0, s1): the output (dst null, whole K) or the
// tile-local fp32 partial at dst (always, when PART_ONLY).
template <bool A_FQ, bool PART_ONLY = false, bool TW = false>
__device__ __forceinline__ void gemm_tile_run(const GemmArgs& g, char* lds, int lin, int s0,
                                              int s1, float* dst) {
  int tm, tn;
  gemm_tile_of(lin, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t K = g.K;
  const int64_t k_lo = (int64_t)s0 * BK;
  const int64_t k_len = min((int64_t)s1 * BK, K) - k_lo;
  const int t = threadIdx.x;

  // sources (rows past M or N are clamped to the last one; never stored)
  GemmSrc src;
  // (K ranges start at multiples of 64, so pointers stay aligned)
  const uint8_t* a_tile_base = reinterpret_cast<const uint8_t*>(g.a + m0 * K + k_lo);
  {
    const int64_t n = min(n0 + (t >> 1), g.N - 1);
    const int64_t wr = g.row_idx ? (int64_t)g.row_idx[n] : n;
    if constexpr (TW)
      gemm_src_tiled_row(src, g.wc, wr, K, k_lo);
    else
      gemm_src_nvfp4_row(src, g.wc, g.ws, wr, K, k_lo);
    if constexpr (A_FQ) {
      const int64_t ar = min(m0 + (t >> 1), g.M - 1);
      src.ar = g.a + ar * K + k_lo + 32 * (t & 1);
    }
  }
  if constexpr (!A_FQ)
    gemm_src_bf16(src, [&](int r) { return min(m0 + r, g.M - 1) - m0; }, K);

  f32x16 acc[kXBlocks][kWBlocks];
  gemm_zero_acc(acc);
  gemm_mainloop<A_FQ, false, TW>(acc, lds, src, a_tile_base, k_len);

  // acc[i][j] = y^T block (n-block j, m-block i): register e of lane l is output
  // row i*32 + l%32, column j*32 + 8*(e/4) + 4*(l/32) + e%4 of the wave's part.
  if (PART_ONLY || dst) {  // fp32 partial of this segment, in register order
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i)
#pragma unroll
      for (int j = 0; j < kWBlocks; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reinterpret_cast<f32x4*>(dst)[((i * kWBlocks + j) * 4 + q) * kGemmThreads + t] =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                    acc[i][j][4 * q + 3]};
    return;
  }
  const bool scaled = g.ga || g.gw;
  const float alpha = scaled ? alpha_of(g.ga, g.gw) : 1.0f;
  if (!g.out_f32 && (g.N & 7) == 0) {  // (the output is 16-byte aligned)
    __syncthreads();  // every wave is done with the operand buffers
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i)
#pragma unroll
      for (int j = 0; j < kWBlocks; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
          float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if (scaled) v0 *= alpha, v1 *= alpha, v2 *= alpha, v3 *= alpha;
          stage_put<BN>(lds, gemm_tile_row(i), gemm_tile_col(j, q),
                        u32x2{(uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16),
                              (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16)});
        }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(g.out) + m0 * g.N + n0;
    stage_store<BN>(lds, (int)min((int64_t)BM, g.M - m0), (int)min((int64_t)BN, g.N - n0),
                    [&](int r) { return out + (int64_t)r * g.N; });
    return;
  }
  const bool vec = (g.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < kXBlocks; ++i) {
    const int64_t row = m0 + gemm_tile_row(i);
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < kWBlocks; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + gemm_tile_col(j, q);
        const int64_t off = row * g.N + col;
        float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (scaled) v0 *= alpha, v1 *= alpha, v2 *= alpha, v3 *= alpha;
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
              static_cast<uint16_t*>(g.out)[off + e] = f32_to_bf16_bits(v[e]);
          }
        }
      }
    }
  }
}

// A_FQ: the activations are quantized to NVFP4 and dequantized (exactly the
// W4A4 operand nvfp4_quantize would give) while their tiles are loaded.
//
// Workgroups 0 .. full-1 take the whole-K tiles, XCD-aware: workgroups are
// dispatched round-robin over the 8 XCDs, and XCD x takes the contiguous band
// [x * full/8, (x+1) * full/8) of the tile order.  The workgroups after them
// (dispatched last) share the remaining tiles, which would otherwise leave
// the chip partly idle in a last round: workgroup w of that band takes the
// flattened steps [w F / P, (w + 1) F / P) of those tiles, F = tail * steps,
// banded per XCD the same way, so neighbouring ranges -- pieces of the same
// tiles -- run on one XCD.  SEGS = false: every range lies in one tile (the
// shared round of a launch that also has whole tiles: P = tail * z).
// SEGS = true (a launch of its own, every tile shared): a range may cover
// the end of one tile and the start of the next, run one after the other.
// (The loop over segments would raise the registers of the whole-tile
// kernel, hence two instantiations.)
// TW: tiled weights (tile.hip).
template <bool A_FQ, bool SEGS, bool TW = false>
__global__ void __launch_bounds__(kGemmThreads) k_gemm(GemmArgs g) {
  extern __shared__ char lds[];
  const int b = blockIdx.x;
  if constexpr (!SEGS) {
    // One call site for both kinds of workgroup (one inlined copy of the tile).
    int lin, s0 = 0, s1 = g.steps;
    float* dst = nullptr;
    if (b < g.full) {
      const int per_xcd = g.full / 8;
      lin = (b & 7) * per_xcd + (b >> 3);
      if (lin >= g.tiles_m * g.tiles_n) return;
    } else {
      // P = tail * z: range w is part w % z of tile w / z, steps
      // [seg S / z, (seg + 1) S / z) -- the partition below in 32-bit arithmetic
      const int per_xcd = (g.parts + 7) / 8;
      const int rb = b - g.full;
      const int w = (rb & 7) * per_xcd + (rb >> 3);
      if (w >= g.parts) return;
      const int z = g.max_seg;
      const int tt = w / z, seg = w - tt * z;
      lin = g.full + tt;
      s0 = seg * g.steps / z;
      s1 = (seg + 1) * g.steps / z;
      dst = g.partial + ((int64_t)tt * z + seg) * (BM * BN);
    }
    gemm_tile_run<A_FQ, false, TW>(g, lds, lin, s0, s1, dst);
    return;
  }
  const int per_xcd = (g.parts + 7) / 8;
  const int w = (b & 7) * per_xcd + (b >> 3);
  if (w >= g.parts) return;
  // Workgroup-uniform and < 2^24 (tail <= 256 tiles, steps <= 2^16).
  const int64_t F = (int64_t)g.tail * g.steps;
  int f = (int)((int64_t)w * F / g.parts);
  const int f1 = (int)((int64_t)(w + 1) * F / g.parts);
  bool first = true;
  while (f < f1) {
    const int tt = f / g.steps;
    const int s0 = f - tt * g.steps;
    const int s1 = min(g.steps, s0 + (f1 - f));
    const int seg = w - sk_owner((int64_t)tt * g.steps, F, g.parts);
    if (!first) __syncthreads();  // every wave is done with the last segment's LDS
    first = false;
    gemm_tile_run<A_FQ, true, TW>(g, lds, g.full + tt, s0, s1,
                                  g.partial + ((int64_t)tt * g.max_seg + seg) * (BM * BN));
    f += s1 - s0;
  }
}

// Shared tiles: out = sum over the tile's segments (in K order) of its fp32
// partials.  A workgroup takes 32 rows x 128 columns of a tile: the rows of
// accumulator block i of wave pair wm and the columns of weight half wn, i.e.
// groups (i, j, q) of the 64 lanes of wave 2 wm + wn -- 16 runs of 1 KB of
// the register order.  Each thread reads 4 f32x4 per segment, sums them in K
// order, stages the sums in LDS as [32][128] and the workgroup stores whole
// row runs.  Z = max_seg (a template argument: all loads of a group are
// issued before the adds, so the sum waits one memory latency, not Z).
constexpr int kReduceRows = 32, kReduceCols = 128, kReducePad = 4;
template <int Z>
__global__ void __launch_bounds__(256) k_gemm_reduce(GemmArgs g) {
  __shared__ float st[kReduceRows][kReduceCols + kReducePad];
  const int tail = blockIdx.x >> 4, part = blockIdx.x & 15;
  const int wm = part >> 2, i = (part >> 1) & 1, wn = part & 1;
  int tm, tn;
  gemm_tile_of(g.full + tail, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t F = (int64_t)g.tail * g.steps;
  const int nseg = sk_owner((int64_t)(tail + 1) * g.steps - 1, F, g.parts) -
                   sk_owner((int64_t)tail * g.steps, F, g.parts) + 1;
  const f32x4* p = reinterpret_cast<const f32x4*>(g.partial + (int64_t)tail * g.max_seg * (BM * BN));
  const int lane = threadIdx.x & 63, tt = (2 * wm + wn) * 64 + lane;
  const float alpha = (g.ga || g.gw) ? alpha_of(g.ga, g.gw) : 1.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int jq = 4 * s + (threadIdx.x >> 6);  // (j, q) of this group
    const int grp = (i * kWBlocks + (jq >> 2)) * 4 + (jq & 3);
    const int64_t idx = (int64_t)grp * kGemmThreads + tt;
    f32x4 q[Z];
#pragma unroll
    for (int z = 0; z < Z; ++z)
      q[z] = z < nseg ? p[(int64_t)z * (BM * BN / 4) + idx] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 v = q[0];
#pragma unroll
    for (int z = 1; z < Z; ++z)
      if (z < nseg) v[0] += q[z][0], v[1] += q[z][1], v[2] += q[z][2], v[3] += q[z][3];
    if (g.ga || g.gw) v[0] *= alpha, v[1] *= alpha, v[2] *= alpha, v[3] *= alpha;
    const int c = acc_col(tt, jq >> 2, jq & 3) - wn * 128;
    *reinterpret_cast<f32x4*>(&st[lane & 31][c]) = v;
  }
  __syncthreads();
  // 32 rows x 128 columns: 16 threads per row, 8 columns each, two passes
  const int64_t row0 = (int64_t)tm * BM + wm * 64 + i * 32;
  const int64_t col0 = (int64_t)tn * BN + wn * 128;
  const int c8 = (threadIdx.x & 15) * 8;
  const int64_t col = col0 + c8;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = pass * 16 + (threadIdx.x >> 4);
    const int64_t row = row0 + r;
    if (row >= g.M || col >= g.N) continue;
    const float* v = &st[r][c8];
    const int64_t off = row * g.N + col;
    if ((g.N & 7) == 0 && col + 7 < g.N) {
      if (g.out_f32) {
        float* o = static_cast<float*>(g.out) + off;
        *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
      } else {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pk[e] = (uint32_t)f32_to_bf16_bits(v[2 * e]) |
                  ((uint32_t)f32_to_bf16_bits(v[2 * e + 1]) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.out) + off) = pk;
      }
    } else {
      for (int e = 0; e < 8 && col + e < g.N; ++e) {
        if (g.out_f32)
          static_cast<float*>(g.out)[off + e] = v[e];
        else
          static_cast<uint16_t*>(g.out)[off + e] = f32_to_bf16_bits(v[e]);
      }
    }
  }
}

// Most segments of one tile when T tiles of S steps are shared by P workgroups.
int max_segments(int64_t T, int64_t S, int P) {
  const int64_t F = T * S;
  int m = 0;
  for (int64_t t = 0; t < T; ++t) {
    const int n = sk_owner((t + 1) * S - 1, F, P) - sk_owner(t * S, F, P) + 1;
    if (n > m) m = n;
  }
  return m;
}

}  // namespace

GemmSplitPlan gemm_split_plan(int64_t M, int64_t n_out, int64_t K, int num_cus) {
  // One 256 x 256 tile per CU at a time (128 KB of LDS), so a launch runs in
  // rounds of num_cus tiles.  Whole rounds run unsplit.  The rem tiles of a
  // last, partly filled round are split over K into z = num_cus / rem equal
  // parts (<= 8, >= 8 steps each), so their parts fill that round; their
  // workgroups follow the whole tiles' in the same launch and start as CUs
  // free up.  When there are fewer tiles than CUs, every tile is shared: P
  // workgroups each take an equal contiguous range of all the tiles' K steps
  // (>= 8 steps, <= 8 segments per tile), P from a cost model -- the longest
  // range at about 3.5 TFLOP/s per CU plus the fp32 partials written and read
  // back at about 5 TB/s -- against the unsplit launch.
  GemmSplitPlan p;
  const int64_t tiles = ((M + BM - 1) / BM) * ((n_out + BN - 1) / BN);
  const int64_t steps = (K + BK - 1) / BK;
  p.full = tiles;
  p.tail = 0;
  p.parts = 0;
  p.max_seg = 0;
  p.own_launch = false;
  if (tiles >= num_cus) {
    const int64_t rem = tiles % num_cus;
    if (rem == 0) return p;
    int64_t z = num_cus / rem;
    if (z > steps / kMinSegSteps) z = steps / kMinSegSteps;
    if (z > kMaxGemmSegs) z = kMaxGemmSegs;
    if (z < 2) return p;
    p.full = tiles - rem;
    p.tail = rem;
    p.parts = (int)(rem * z);
    p.max_seg = (int)z;
    return p;
  }
  const double step_s = 2.0 * BM * BN * BK / 3.5e12;
  const double seg_s = 2.0 * BM * BN * 4.0 / 5.0e12;
  const int64_t F = tiles * steps;
  auto cost = [&](int64_t P) {
    const double span = (double)((F + P - 1) / P) * step_s;
    return P > tiles ? span + (double)(P + tiles) * seg_s : span;
  };
  int64_t best = tiles;
  double best_cost = 0.95 * cost(tiles);  // splitting must gain 5%
  const int64_t pmax = std::min<int64_t>(num_cus, F / kMinSegSteps);
  for (int64_t P = tiles + 1; P <= pmax; ++P) {
    const double c = cost(P);
    if (c < best_cost && max_segments(tiles, steps, (int)P) <= kMaxGemmSegs) {
      best = P;
      best_cost = c;
    }
  }
  if (best > tiles) {
    p.full = 0;
    p.tail = tiles;
    p.parts = (int)best;
    p.max_seg = max_segments(tiles, steps, (int)best);
    p.own_launch = true;
  }
  return p;
}

size_t gemm_workspace_bytes(int64_t M, int64_t n_out, int64_t K, int num_cus) {
  const GemmSplitPlan p = gemm_split_plan(M, n_out, K, num_cus);
  return p.parts > 0 ? (size_t)p.tail * (size_t)p.max_seg * BM * BN * sizeof(float) : 0;
}

int launch_gemm(GemmA mode, const void* a, int64_t M, int64_t K, const uint8_t* wc,
                const uint8_t* ws, const int32_t* row_idx, int64_t n_out, bool out_f32, void* out,
                void* workspace, hipStream_t stream, Alpha alpha, bool tiled) {
  // activation offsets inside a 256-row tile are 32-bit byte offsets (the
  // entry points reject a longer K before launching)
  if (K > ((int64_t)1 << 22)) return -1;
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(a);
  g.wc = wc;
  g.ws = ws;
  g.row_idx = row_idx;
  g.out = out;
  g.M = M;
  g.N = n_out;
  g.K = K;
  g.out_f32 = out_f32 ? 1 : 0;
  g.ga = alpha.a;
  g.gw = alpha.w;
  g.tiles_m = (int)((M + BM - 1) / BM);
  g.tiles_n = (int)((n_out + BN - 1) / BN);
  g.steps = (int)((K + BK - 1) / BK);
  const GemmSplitPlan p = gemm_split_plan(M, n_out, K, kNumCUs);
  g.full = (int)p.full;
  g.tail = (int)p.tail;
  g.parts = p.parts;
  g.max_seg = p.max_seg;
  if (g.parts > 0 && !workspace) return -1;
  if (g.parts == 0) {
    g.full = g.tiles_m * g.tiles_n;  // every tile whole
    g.tail = 0;
  }
  g.partial = static_cast<float*>(workspace);
  // The bands need a multiple of 8 workgroups (the XCD banding): a split
  // plan's `full` is a multiple of the CU count (or 0); an unsplit one is
  // padded and the extra workgroups exit, as do those past the last range.
  if (g.full % 8 != 0) g.full = (g.full + 7) / 8 * 8;
  const bool fq = mode == GemmA::kFakeQuant;
  const int64_t grid = g.full + ((int64_t)g.parts + 7) / 8 * 8;
  if (grid > INT32_MAX) return -1;
  // (Both activation modes take the same partition, so the fused-quantizer
  // product stays bit-identical to quantize + the W4A4 GEMM.)
  if (tiled) {  // (bf16 activations only)
    if (fq) return -1;
    if (p.own_launch)
      hipLaunchKernelGGL((k_gemm<false, true, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                         kLdsBytes, stream, g);
    else
      hipLaunchKernelGGL((k_gemm<false, false, true>), dim3((unsigned)grid),
                         dim3(kGemmThreads), kLdsBytes, stream, g);
  } else if (p.own_launch) {
    if (fq)
      hipLaunchKernelGGL((k_gemm<true, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                         kLdsBytes, stream, g);
    else
      hipLaunchKernelGGL((k_gemm<false, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                         kLdsBytes, stream, g);
  } else {
    if (fq)
      hipLaunchKernelGGL((k_gemm<true, false>), dim3((unsigned)grid), dim3(kGemmThreads),
                         kLdsBytes, stream, g);
    else
      hipLaunchKernelGGL((k_gemm<false, false>), dim3((unsigned)grid), dim3(kGemmThreads),
                         kLdsBytes, stream, g);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  if (g.parts > 0) {
    const dim3 rg((unsigned)(g.tail * 16));
    switch (g.max_seg) {
      case 1: hipLaunchKernelGGL(k_gemm_reduce<1>, rg, dim3(256), 0, stream, g); break;
      case 2: hipLaunchKernelGGL(k_gemm_reduce<2>, rg, dim3(256), 0, stream, g); break;
      case 3: hipLaunchKernelGGL(k_gemm_reduce<3>, rg, dim3(256), 0, stream, g); break;
      case 4: hipLaunchKernelGGL(k_gemm_reduce<4>, rg, dim3(256), 0, stream, g); break;
      case 5: hipLaunchKernelGGL(k_gemm_reduce<5>, rg, dim3(256), 0, stream, g); break;
      case 6: hipLaunchKernelGGL(k_gemm_reduce<6>, rg, dim3(256), 0, stream, g); break;
      case 7: hipLaunchKernelGGL(k_gemm_reduce<7>, rg, dim3(256), 0, stream, g); break;
      case 8: hipLaunchKernelGGL(k_gemm_reduce<8>, rg, dim3(256), 0, stream, g); break;
      default: return -2;
    }
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace nvfp4
