// moe.hip -- routed mixture-of-experts pieces of the NVFP4 linear layer.
//
// The pages' MoE model routes every token to a few experts out of many
// ("What 350+ Experiments Taught Us About Serving Qwen 3.6 35B-A3B", section 1)
// and runs its NVFP4 experts through a grouped kernel (section 7).  The layer
// is built from three device steps on one stream, with no host round trip:
//   align    -- stable counting sort of (token, slot) assignments by expert;
//   grouped  -- per-expert W4A16 GEMM over the gathered rows, with a SwiGLU
//               (gate+up) or a per-row scale (gate weight) epilogue: a
//               weight-streaming GEMV kernel (16 rows of one expert per
//               workgroup) when experts get few rows, the 256 x 256 MFMA tile
//               of gemm_core.h when they get many;
//   combine  -- per-token sum of its slots' outputs.
#include "gemm_core.h"
#include "gemv_core.h"
#include "moe.h"

namespace nvfp4 {

namespace {

constexpr int kAlignBlock = 256;  // assignments per align workgroup

// ---- align: block histograms -> per-(block, expert) bases -> ranked scatter ----

// Entries of sid[base .. p) equal to e (base 16-byte aligned): 16-byte LDS
// reads, several in flight, instead of one dependent read per entry.  With G
// threads per entry, thread g of them counts the 4-entry groups g, g + G, ...
// (and g = 0 the last partial group); their counts add up to the total.
__device__ __forceinline__ int count_before(const int* sid, int base, int p, int e, int g = 0,
                                            int G = 1) {
  const int n = p - base, n4 = n >> 2;
  const int4* v = reinterpret_cast<const int4*>(sid + base);
  int r = 0;
#pragma unroll 4
  for (int j = g; j < n4; j += G) {
    const int4 x = v[j];
    r += (x.x == e) + (x.y == e) + (x.z == e) + (x.w == e);
  }
  if (g == 0)
    for (int q = 4 * n4; q < n; ++q) r += sid[base + q] == e;
  return r;
}

__global__ void __launch_bounds__(256) k_align_hist(const int32_t* __restrict__ ids, int64_t R,
                                                    int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMoeMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kAlignBlock + threadIdx.x;
  if (p < R) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);  // integer counts: order-free
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads.  offsets = exclusive scan of the expert
// totals; hist[b][e] is replaced by the first row of expert e owned by block b.
// Expert offsets and, for every (block, expert), the first row that block's
// assignments of that expert land in.  The 1024 threads split each expert's
// column of per-block counts into `slices` contiguous ranges (slices * ep2 =
// 1024, ep2 = E rounded up to a power of two), so every thread walks at most
// ceil(nblocks / slices) blocks, 8 independent loads at a time.
__global__ void __launch_bounds__(1024) k_align_scan(int32_t* __restrict__ hist, int nblocks,
                                                     int E, int ep2,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int part[kMoeMaxExperts];  // [slice][expert] partial sums, then prefixes
  __shared__ int tot[kMoeMaxExperts];
  const int slices = kMoeMaxExperts / ep2;
  const int e = threadIdx.x % ep2, sl = threadIdx.x / ep2;
  const int per = (nblocks + slices - 1) / slices;
  const int b0 = min(sl * per, nblocks), b1 = min(b0 + per, nblocks);
  int sum = 0;
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = hist[(int64_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += h[i];
    }
    for (; b < b1; ++b) sum += hist[(int64_t)b * E + e];
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  // expert totals, and each slice's exclusive prefix within its expert
  if (sl == 0) {
    int run = 0;
    for (int j = 0; j < slices; ++j) {
      const int v = part[j * ep2 + e];
      part[j * ep2 + e] = run;
      run += v;
    }
    tot[e] = e < E ? run : 0;
  } else {
    tot[threadIdx.x] = 0;  // slots past ep2 hold no expert
  }
  __syncthreads();
  // inclusive Hillis-Steele scan of the expert totals over 1024 slots
  const int t = threadIdx.x;
  for (int d = 1; d < kMoeMaxExperts; d <<= 1) {
    const int v = t >= d ? tot[t - d] : 0;
    __syncthreads();
    tot[t] += v;
    __syncthreads();
  }
  if (e < E) {
    const int excl = (e > 0 ? tot[e - 1] : 0);
    if (sl == 0) offsets[e] = excl;
    int run = excl + part[sl * ep2 + e];
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = hist[(int64_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hist[(int64_t)(b + i) * E + e] = run;
        run += h[i];
      }
    }
    for (; b < b1; ++b) {
      const int h = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = run;
      run += h;
    }
  }
  if (t == 0) offsets[E] = tot[E - 1];
}

__global__ void __launch_bounds__(256) k_align_scatter(const int32_t* __restrict__ ids,
                                                       const float* __restrict__ gates,
                                                       int64_t R, int topk, int E,
                                                       const int32_t* __restrict__ base,
                                                       int32_t* __restrict__ gather_idx,
                                                       int32_t* __restrict__ slot_pos,
                                                       float* __restrict__ row_gates) {
  __shared__ __attribute__((aligned(16))) int sid[kAlignBlock];
  const int i = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * kAlignBlock + i;
  sid[i] = p < R ? ids[p] : -1;
  __syncthreads();
  if (p >= R) return;
  const int e = sid[i];
  if (e < 0 || e >= E) return;
  const int rank = count_before(sid, 0, i, e);  // earlier assignments, same expert
  const int dest = base[(int64_t)blockIdx.x * E + e] + rank;
  gather_idx[dest] = (int32_t)(p / topk);
  slot_pos[p] = dest;
  if (gates) row_gates[dest] = gates[p];
}

// SwiGLU of one output: silu(g) * u = g / (1 + e^-g) * u, in fp32 with the
// hardware exponential and reciprocal (a few ulp of fp32, far below the bf16
// rounding of the stored result).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __frcp_rn(1.0f + __expf(-g)) * u;
}

// ---- grouped GEMV -------------------------------------------------------------

constexpr int kGroupRows = 16;  // rows of one expert per workgroup (one 16-row MFMA tile)
constexpr int kGroupWaves = 4;

struct GroupedArgs {
  const uint16_t* a;
  const int32_t* gather;
  const int32_t* offsets;
  const uint8_t* wc;  // row-major codes [E][N][K/2], or the tiled experts (k_grouped_gemv<TR, true>)
  const uint8_t* ws;
  const float* wg;  // per-expert global scales [E] of two-level weights, or NULL
  const float* row_scale;
  uint16_t* out;
  int64_t K;
  int64_t N;
  int E;
  int steps;
  int swiglu;
};

// Find (expert, chunk) of workgroup `bx` in the device-side schedule where
// expert e owns ceil(rows_e / chunk_rows) consecutive chunks, and the chunk's
// first grouped row r0 and its row count.  Wave-uniform.  The offsets of up
// to 256 experts are loaded in one round (one memory latency, not one per 64
// experts plus one more for the chunk's rows).
struct ChunkPos {
  int e, c, rows;
  int64_t r0;
};
__device__ __forceinline__ bool find_chunk(const int32_t* offsets, int E, int bx, int chunk_rows,
                                           ChunkPos& pos) {
  constexpr int kRound = 4;  // 64-expert groups per round of loads
  const int lane = threadIdx.x & 63;
  int run = 0;
  for (int base = 0; base < E; base += 64 * kRound) {
    int lo[kRound], hi[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int e = base + 64 * u + lane;
      lo[u] = e < E ? offsets[e] : 0;
      hi[u] = e < E ? offsets[e + 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int gb = base + 64 * u;
      if (gb >= E) return false;
      const int ch = gb + lane < E ? (hi[u] - lo[u] + chunk_rows - 1) / chunk_rows : 0;
      int inc = ch;  // inclusive prefix over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d, 64);
        if (lane >= d) inc += v;
      }
      const int total = __shfl(inc, 63, 64);
      if (bx < run + total) {
        const unsigned long long hit = __ballot(run + inc > bx);
        const int l = __builtin_ctzll(hit);
        pos.e = gb + l;
        pos.c = bx - run - (__shfl(inc, l, 64) - __shfl(ch, l, 64));
        pos.r0 = (int64_t)__shfl(lo[u], l, 64) + (int64_t)pos.c * chunk_rows;
        pos.rows = (int)min((int64_t)__shfl(hi[u], l, 64) - pos.r0, (int64_t)chunk_rows);
        return true;
      }
      run += total;
    }
  }
  return false;
}

// One workgroup: up to 16 grouped rows of one expert (staged in LDS) against
// kGroupWaves weight tiles (SWIGLU: tile pairs gate/up) of that expert.
template <int TR, bool TL = false, int NW = kGroupWaves>
__global__ void __launch_bounds__(64 * NW) k_grouped_gemv(GroupedArgs g) {
  extern __shared__ uint16_t xs[];  // [kGroupRows][lds_x_stride(steps)]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15, q = lane >> 4;
  const int64_t K = g.K;

  ChunkPos pos;
  if (!find_chunk(g.offsets, g.E, blockIdx.x, kGroupRows, pos)) return;  // uniform
  const int e = pos.e, rows = pos.rows;
  const int64_t r0 = pos.r0;
  const uint16_t* a = g.a;
  const int32_t* gather = g.gather;
  const int stride = lds_x_stride(g.steps);
  stage_activations(xs, rows, 0, g.steps * kGemvStep, stride, K, [a, gather, r0, K](int m) {
    const int64_t r = r0 + m;
    return a + (int64_t)(gather ? gather[r] : r) * K;
  });

  // weight rows: NONE -> tiles (blockIdx.y*nw + wave)*TR + t; SWIGLU (TR == 2) ->
  // gate tile blockIdx.y*nw + wave and the matching up tile N/2 further.
  const int64_t gt = (int64_t)blockIdx.y * NW + wave;
  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
  if constexpr (TL) {  // expert e's N / 16 tiles of g.steps blocks
    const uint8_t* we = g.wc + (int64_t)e * (g.N / 16) * g.steps * 2304;
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      int64_t tile = g.swiglu ? (int64_t)t * (g.N / 32) + gt : gt * TR + t;
      if (tile >= g.N / 16) tile = g.N / 16 - 1;  // padding tile: never stored
      cptr[t] = we + tile * g.steps * 2304 + 16 * lane;
      sptr[t] = we + tile * g.steps * 2304 + 2048 + 4 * lane;
    }
  } else {
    const uint8_t* we_c = g.wc + (int64_t)e * g.N * (K / 2);
    const uint8_t* we_s = g.ws + (int64_t)e * g.N * (K / 16);
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      int64_t n = g.swiglu ? (int64_t)t * (g.N / 2) + gt * 16 + ln : (gt * TR + t) * 16 + ln;
      if (n >= g.N) n = g.N - 1;  // padding column: never stored
      cptr[t] = we_c + n * (K / 2);
      sptr[t] = we_s + n * (K / 16);
    }
  }
  const uint16_t* xl[1] = {xs + min(ln, rows - 1) * stride + 64 * q};

  f32x4 acc[TR][1];
#pragma unroll
  for (int t = 0; t < TR; ++t) acc[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemv_accumulate<1, TR, TL>(acc, cptr, sptr, xl, K, 0, g.steps,
                             TL ? g.steps : (int)(K / kGemvStep));

  // lane holds C[m = 4*q + r][column 16*tile + ln]; the sums are h / g_e
  const float ge = g.wg ? g.wg[e] : 1.0f;
  const int64_t width = g.swiglu ? g.N / 2 : g.N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m >= rows) continue;
    const int64_t row = r0 + m;
    const float rs = g.row_scale ? g.row_scale[row] : 1.0f;
    if (g.swiglu) {
      const int64_t col = gt * 16 + ln;
      if (col < width) {
        const float hg = acc[0][0][r] * ge, hu = acc[TR - 1][0][r] * ge;
        float v = silu_mul(hg, hu);
        if (g.row_scale) v *= rs;
        g.out[row * width + col] = f32_to_bf16_bits(v);
      }
    } else {
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        const int64_t col = (gt * TR + t) * 16 + ln;
        if (col < width) {
          float v = acc[t][0][r] * ge;
          if (g.row_scale) v *= rs;
          g.out[row * width + col] = f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// ---- grouped MFMA GEMM (many rows per expert) ---------------------------------

struct GroupedMfmaArgs {
  const uint16_t* a;
  const int32_t* gather;
  const int32_t* offsets;
  const uint8_t* wc;  // row-major codes [E][N][K/2], or the tiled experts (k_grouped_mfma<true>)
  const uint8_t* ws;
  const float* wg;  // per-expert global scales [E] of two-level weights, or NULL
  const float* row_scale;
  uint16_t* out;
  int64_t K;
  int64_t N;
  int E;
  int swiglu;
  int n_tiles;  // tiles per chunk: ceil(N / 256), or ceil(N/2 / 128) with SWIGLU
  int chunks;   // upper bound of the 256-row chunks
};

// One workgroup: one 256-row chunk of one expert's gathered rows against one
// tile of that expert's weight rows.  Workgroups beyond the schedule (the grid
// is sized for the worst case) return at once.  SWIGLU tiles hold, for 128
// outputs o0 .. o0+127, gate rows o0 + h*64 + u and up rows N/2 + o0 + h*64 + u
// (h = 0, 1; u < 64) at tile columns 128 h + u and 128 h + 64 + u: each gate
// accumulator and its up partner sit in the same lane and register (blocks j
// and j + 2 of the wave), so the epilogue needs no exchange.
template <bool TW>
__global__ void __launch_bounds__(kGemmThreads) k_grouped_mfma(GroupedMfmaArgs g) {
  extern __shared__ char lds[];
  // Consecutive workgroups go to consecutive XCDs.  Chunk c runs on XCD c % 8,
  // its n_tiles tiles one after another there, so they share its activation
  // rows in one L2; and the chunks that exist (the host knows only an upper
  // bound) spread evenly over the XCDs, the surplus workgroups at the end of
  // every XCD's sequence.
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int chunk = (k / g.n_tiles) * 8 + xcd, tn = k % g.n_tiles;
  if (chunk >= g.chunks) return;
  ChunkPos pos;
  if (!find_chunk(g.offsets, g.E, chunk, BM, pos)) return;  // uniform over the workgroup
  const int e = pos.e, rows = pos.rows;
  const int64_t r0 = pos.r0;
  const int64_t K = g.K, N = g.N, half_n = N / 2;
  const int t = threadIdx.x;

  // The gathered row indices of this thread's activation copies (rows past
  // the chunk repeat its last row) are loaded now and used only after the
  // first weight loads are issued; the epilogue's row and expert scales are
  // loaded now too, so no memory latency is left at either end of the tile.
  int64_t arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + min(gemm_copy_row(i), rows - 1);
    arow[i] = g.gather ? (int64_t)g.gather[r] : r;
  }
  float rs[kXBlocks];
#pragma unroll
  for (int i = 0; i < kXBlocks; ++i) {
    const int tr = gemm_tile_row(i);
    rs[i] = g.row_scale && tr < rows ? g.row_scale[r0 + tr] : 1.0f;
  }
  const float ge = g.wg ? g.wg[e] : 1.0f;  // the sums are h / g_e

  GemmSrc src;
  // row-major: expert e's rows; tiled: its N / 16 tiles of ceil(K / 256) blocks
  const uint8_t* we_c = TW ? g.wc + (int64_t)e * (N / 16) * ((K + 255) / 256) * 2304
                           : g.wc + (int64_t)e * N * (K / 2);
  const uint8_t* we_s = TW ? nullptr : g.ws + (int64_t)e * N * (K / 16);
  {
    const int row = t >> 1;  // tile row u + 128 q
    const int q = row >> 7, u = row & 127;
    int64_t n;
    if (g.swiglu) {
      const int64_t o = min((int64_t)tn * 128 + q * 64 + (u & 63), half_n - 1);
      n = u < 64 ? o : half_n + o;
    } else {
      n = min((int64_t)tn * BN + row, N - 1);
    }
    if constexpr (TW)
      gemm_src_tiled_row(src, we_c, n, K, 0);
    else
      gemm_src_nvfp4_row(src, we_c, we_s, n, K, 0);
  }

  f32x16 acc[kXBlocks][kWBlocks];
  gemm_zero_acc(acc);
  // (an expert's last chunk is partly filled: waves skip the 32-row blocks past it)
  gemm_mainloop<false, true, TW>(acc, lds, src, reinterpret_cast<const uint8_t*>(g.a), K, rows,
                             [&](GemmSrc& s) { gemm_src_bf16_rows(s, arow, K); });

  // Staged output (N % 16 == 0 and a 16-byte aligned output: every row run is
  // aligned); the blocks past the chunk's rows are not written.
  __syncthreads();  // every wave is done with the operand buffers
  const int wn = (t >> 6) & 1, h = (t & 63) >> 5;
  if (g.swiglu) {
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i) {
      const int tr = gemm_tile_row(i);
      if (tr >= rows) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t pk[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            float v[2];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const float hg = acc[i][j][4 * q + 2 * p + w] * ge;
              const float hu = acc[i][j + 2][4 * q + 2 * p + w] * ge;
              v[w] = silu_mul(hg, hu);
              if (g.row_scale) v[w] *= rs[i];
            }
            pk[p] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
          }
          stage_put<BN / 2>(lds, tr, wn * 64 + j * 32 + 8 * q + 4 * h, u32x2{pk[0], pk[1]});
        }
      }
    }
    __syncthreads();
    uint16_t* out = g.out + r0 * half_n + (int64_t)tn * 128;
    stage_store<BN / 2>(lds, rows, (int)min((int64_t)128, half_n - (int64_t)tn * 128),
                        [&](int r) { return out + (int64_t)r * half_n; });
  } else {
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i) {
      const int tr = gemm_tile_row(i);
      if (tr >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t pk[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            float v0 = acc[i][j][4 * q + 2 * p] * ge, v1 = acc[i][j][4 * q + 2 * p + 1] * ge;
            if (g.row_scale) v0 *= rs[i], v1 *= rs[i];
            pk[p] = (uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
          }
          stage_put<BN>(lds, tr, gemm_tile_col(j, q), u32x2{pk[0], pk[1]});
        }
      }
    }
    __syncthreads();
    uint16_t* out = g.out + r0 * N + (int64_t)tn * BN;
    stage_store<BN>(lds, rows, (int)min((int64_t)BN, N - (int64_t)tn * BN),
                    [&](int r) { return out + (int64_t)r * N; });
  }
}

// ---- combine --------------------------------------------------------------------

__global__ void __launch_bounds__(256) k_moe_combine(const uint16_t* __restrict__ y,
                                                     const int32_t* __restrict__ slot_pos,
                                                     int64_t T, int topk, int64_t H,
                                                     uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (token, 8 columns)
  const int64_t per_row = H / 8;
  if (i >= T * per_row) return;
  const int64_t t = i / per_row, c8 = (i - t * per_row) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const u32x4& v) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s[2 * w] += bf16_bits_to_f32(v[w] & 0xFFFFu);
      s[2 * w + 1] += bf16_bits_to_f32(v[w] >> 16);
    }
  };
  int j = 0;
  // eight slots at a time: their rows, then all eight row loads in flight,
  // then the adds in slot order
  for (; j + 8 <= topk; j += 8) {
    int64_t rows[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) rows[u] = slot_pos[t * topk + j + u];
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const u32x4*>(y + rows[u] * H + c8);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(v[u]);
  }
  for (; j < topk; ++j)
    add(*reinterpret_cast<const u32x4*>(y + (int64_t)slot_pos[t * topk + j] * H + c8));
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    o[w] = (uint32_t)f32_to_bf16_bits(s[2 * w]) | ((uint32_t)f32_to_bf16_bits(s[2 * w + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + t * H + c8) = o;
}

// Small batches (R <= 2048 assignments, a decode step): the same three phases
// in one workgroup of 1024 threads, through LDS, with the same result (the
// per-(block, expert) bases and the in-block ranks define one stable order).
// The ids and gates are read together at the start (one memory latency), the
// expert totals are scanned by wave shuffles (two barriers), and up to four
// threads share the ranking of one entry when there are threads to spare.
constexpr int kAlignSmallMax = 2048;

__global__ void __launch_bounds__(1024) k_align_small(const int32_t* __restrict__ ids,
                                                      const float* __restrict__ gates, int R,
                                                      int topk, int E,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ gather_idx,
                                                      int32_t* __restrict__ slot_pos,
                                                      float* __restrict__ row_gates) {
  __shared__ __attribute__((aligned(16))) int sid[kAlignSmallMax];
  __shared__ float sg[kAlignSmallMax];
  __shared__ int hist[(kAlignSmallMax / kAlignBlock) * kMoeMaxExperts];
  __shared__ int wsum[kMoeMaxExperts / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nb = (R + kAlignBlock - 1) / kAlignBlock;
  for (int p = t; p < R; p += blockDim.x) {
    sid[p] = ids[p];
    if (gates) sg[p] = gates[p];
  }
  for (int i = t; i < nb * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int p = t; p < R; p += blockDim.x) {
    const int e = sid[p];
    if (e >= 0 && e < E) atomicAdd(&hist[(p / kAlignBlock) * E + e], 1);
  }
  __syncthreads();
  int total = 0;  // thread t < E: expert t's prefix over blocks
  if (t < E)
    for (int b = 0; b < nb; ++b) {
      const int h = hist[b * E + t];
      hist[b * E + t] = total;
      total += h;
    }
  // inclusive scan of the totals over the threads: within each wave, then
  // the sums of the waves before it
  int inc = total;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d, 64);
    if (lane >= d) inc += v;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wsum[w];
  if (t < E) {
    const int excl = inc - total;
    offsets[t] = excl;
    for (int b = 0; b < nb; ++b) hist[b * E + t] += excl;
  }
  if (t == E - 1) offsets[E] = inc;
  __syncthreads();
  // G neighbouring threads rank entry p; their partial counts meet in lane g = 0
  const int lg = R <= 256 ? 2 : (R <= 512 ? 1 : 0), G = 1 << lg;
  for (int i = t; i < (R << lg); i += blockDim.x) {
    const int p = i >> lg, g = i & (G - 1);
    const int e = sid[p];
    const bool valid = e >= 0 && e < E;
    const int b = p / kAlignBlock;
    int r = valid ? count_before(sid, b * kAlignBlock, p, e, g, G) : 0;
    for (int o = 1; o < G; o <<= 1) r += __shfl_xor(r, o, 64);
    if (valid && g == 0) {
      const int dest = hist[b * E + e] + r;
      gather_idx[dest] = p / topk;
      slot_pos[p] = dest;
      if (gates) row_gates[dest] = sg[p];
    }
  }
}

}  // namespace

size_t moe_align_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  const int64_t R = T * topk;
  const int64_t nb = (R + kAlignBlock - 1) / kAlignBlock;
  return (size_t)nb * (size_t)E * sizeof(int32_t);
}

int launch_moe_align(const int32_t* ids, const float* gates, int64_t T, int64_t topk, int64_t E,
                     int32_t* offsets, int32_t* gather_idx, int32_t* slot_pos, float* row_gates,
                     void* workspace, hipStream_t stream) {
  const int64_t R = T * topk;
  if (R <= kAlignSmallMax) {  // one launch instead of three
    hipLaunchKernelGGL(k_align_small, dim3(1), dim3(kMoeMaxExperts), 0, stream, ids, gates,
                       (int)R, (int)topk, (int)E, offsets, gather_idx, slot_pos, row_gates);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int nb = (int)((R + kAlignBlock - 1) / kAlignBlock);
  int32_t* hist = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(k_align_hist, dim3(nb), dim3(kAlignBlock), 0, stream, ids, R, (int)E, hist);
  int ep2 = 1;
  while (ep2 < E) ep2 <<= 1;
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(kMoeMaxExperts), 0, stream, hist, nb, (int)E,
                     ep2, offsets);
  hipLaunchKernelGGL(k_align_scatter, dim3(nb), dim3(kAlignBlock), 0, stream, ids, gates, R,
                     (int)topk, (int)E, hist, gather_idx, slot_pos, row_gates);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

size_t moe_grouped_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K) {
  (void)R;
  (void)E;
  (void)N;
  (void)K;
  return 0;
}

// LDS of the grouped GEMV: kGroupRows activation rows of the whole K range.
static size_t grouped_gemv_lds_bytes(int64_t K) {
  const int steps = (int)((K + kGemvStep - 1) / kGemvStep);
  return (size_t)kGroupRows * lds_x_stride(steps) * sizeof(uint16_t);
}

GroupedPath grouped_path(int64_t a_rows, int64_t K, int64_t E, int64_t R,
                         const PlanOverride& ov) {
  // MFMA tiles once experts average enough rows to fill them (32 by default);
  // the GEMV stages the rows' whole K range in LDS, so a K past what LDS holds
  // (above 4,864) runs the MFMA kernel at any row count.  The MFMA kernel's
  // activation offsets are 32-bit.
  const int64_t min_avg = ov.grouped_mfma_min_rows >= 0 ? ov.grouped_mfma_min_rows : 32;
  const bool mfma_fits = a_rows * K * 2 < ((int64_t)1 << 32);
  const bool gemv_fits = grouped_gemv_lds_bytes(K) <= kGroupedGemvMaxLds;
  if (mfma_fits && (R >= min_avg * E || !gemv_fits)) return GroupedPath::kMfma;
  if (gemv_fits) return GroupedPath::kGemv;
  return GroupedPath::kNone;
}

int launch_grouped_gemm(const uint16_t* a, int64_t a_rows, int64_t K, const int32_t* gather,
                        const int32_t* offsets, int64_t E, int64_t R, int64_t N,
                        const uint8_t* wc, const uint8_t* ws, const float* wg,
                        const float* row_scale, bool swiglu, uint16_t* out, void* workspace,
                        hipStream_t stream, const PlanOverride& ov, bool tiled) {
  (void)workspace;
  const GroupedPath path = grouped_path(a_rows, K, E, R, ov);
  if (path == GroupedPath::kNone) return -2;
  if (path == GroupedPath::kMfma) {
    GroupedMfmaArgs m;
    m.a = a;
    m.gather = gather;
    m.offsets = offsets;
    m.wc = wc;
    m.ws = ws;
    m.wg = wg;
    m.row_scale = row_scale;
    m.out = out;
    m.K = K;
    m.N = N;
    m.E = (int)E;
    m.swiglu = swiglu ? 1 : 0;
    m.n_tiles = (int)(swiglu ? (N / 2 + 127) / 128 : (N + BN - 1) / BN);
    const int64_t chunks = (R + BM - 1) / BM + E;  // upper bound
    m.chunks = (int)chunks;
    const int grid = (int)(((chunks + 7) / 8) * 8 * m.n_tiles);
    if (tiled)
      hipLaunchKernelGGL(k_grouped_mfma<true>, dim3(grid), dim3(kGemmThreads), kLdsBytes, stream,
                         m);
    else
      hipLaunchKernelGGL(k_grouped_mfma<false>, dim3(grid), dim3(kGemmThreads), kLdsBytes,
                         stream, m);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  GroupedArgs g;
  g.a = a;
  g.gather = gather;
  g.offsets = offsets;
  g.wc = wc;
  g.ws = ws;
  g.wg = wg;
  g.row_scale = row_scale;
  g.out = out;
  g.K = K;
  g.N = N;
  g.E = (int)E;
  g.steps = (int)((K + kGemvStep - 1) / kGemvStep);  // including a partial last step
  g.swiglu = swiglu ? 1 : 0;
  const int64_t chunks = (R + kGroupRows - 1) / kGroupRows + E;  // upper bound
  const int64_t tiles_y = swiglu ? (N / 2 + 15) / 16 : (N + 31) / 32;  // gate tiles or tile pairs
  const size_t lds = grouped_gemv_lds_bytes(K);
  // Tiled experts with a long K (staged rows over 48 KB of LDS, so few
  // workgroups fit a CU): 8 waves share each staged copy (measured at T = 32:
  // gate/up 36.1 -> 34.5 us; row-major experts and the down projection are
  // faster with 4)
  const int nw = ov.grouped_gemv_waves > 0 ? ov.grouped_gemv_waves
                 : (tiled && lds > 48 * 1024) ? 8
                                               : kGroupWaves;
  const int64_t ytiles = (tiles_y + nw - 1) / nw;
  const dim3 grid((unsigned)chunks, (unsigned)ytiles);
  if (tiled) {
    if (nw == 16)
      hipLaunchKernelGGL((k_grouped_gemv<2, true, 16>), grid, dim3(1024), lds, stream, g);
    else if (nw == 8)
      hipLaunchKernelGGL((k_grouped_gemv<2, true, 8>), grid, dim3(512), lds, stream, g);
    else
      hipLaunchKernelGGL((k_grouped_gemv<2, true, 4>), grid, dim3(256), lds, stream, g);
  } else {
    if (nw == 16)
      hipLaunchKernelGGL((k_grouped_gemv<2, false, 16>), grid, dim3(1024), lds, stream, g);
    else if (nw == 8)
      hipLaunchKernelGGL((k_grouped_gemv<2, false, 8>), grid, dim3(512), lds, stream, g);
    else
      hipLaunchKernelGGL((k_grouped_gemv<2, false, 4>), grid, dim3(256), lds, stream, g);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_moe_combine(const uint16_t* y, const int32_t* slot_pos, int64_t T, int64_t topk,
                       int64_t H, uint16_t* out, hipStream_t stream) {
  const int64_t n = T * (H / 8);
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y,
                     slot_pos, T, (int)topk, H, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
