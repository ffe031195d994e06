// topk.hip -- draft proposal from the masked head: top-k of each row of fp32
// logits, best first.
//
// The draft head proposes tokens only from the kept (ranked) rows of the
// vocabulary ("Serving Qwen3.8-27B in 4-bit with a masked speculative decoding
// head", section "The masked head trick").  Order: the larger logit first;
// equal logits by the smaller column (the position in the ranked mask); -0
// below +0.  That order is total, so every element gets a unique 64-bit key
//
//   key = ord(bits(v)) << 32 | (0xFFFFFFFF - column)
//
// where ord maps fp32 bit patterns to unsigned integers in the order of the
// values (sign-magnitude to offset binary), and the top-k are the k largest
// keys.  Every real key is non-zero (the column is < 2^31), so 0 marks an
// empty slot.
//
// Rows longer than one chunk take several levels: each chunk leaves its k best
// keys, and the next level selects from those, until one chunk is left; that
// last level sorts its k keys and writes values and ids.
//
// k <= 64: one wave selects from a chunk of 512 keys (8 per lane) on its own,
// with no LDS traffic and no barriers: the threshold T with exactly k keys
// >= T is built one bit at a time from the top, each trial counted with
// ballots (a 64-lane compare and a popcount per register), stopping as soon
// as a trial leaves exactly k keys above it.
// k > 64: a workgroup selects from a chunk of 2048 keys by radix select, 8
// bits a pass from the top, with 256-bin histograms in LDS; the search stops
// as soon as every key of the bin that holds the k-th largest is needed.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkPer = 8;  // keys per thread
constexpr int kTopkChunk = kTopkThreads * kTopkPer;

__device__ __forceinline__ uint32_t ord_f32(uint32_t u) {
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t unord_f32(uint32_t o) {
  return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
}

struct TopkLevelArgs {
  const float* logits;    // first level: fp32 [M][n_in]
  const uint64_t* keys;   // later levels: keys [M][n_in] (0 = empty slot)
  int64_t n_in;           // elements per row at this level
  int chunks;             // chunks per row at this level
  int k;
  uint64_t* keys_out;     // not last level: [M][chunks][k]
  float* values;          // last level: [M][k]
  int32_t* ids;           // last level: [M][k]
  const int32_t* ids_map; // last level: id = ids_map[column], or the column
  int64_t n_cols;         // columns of the logits (bounds ids_map reads)
};

// Keys of elements i0 + p * STRIDE (p < P) of row m; 0 past the row.  Every
// load is issued (at a clamped index) before any is used, so the P loads are
// in flight together.
template <bool FROM_F32, int P, int STRIDE>
__device__ __forceinline__ void load_keys(const TopkLevelArgs& g, int64_t m, int64_t i0,
                                          uint64_t (&key)[P]) {
  const int64_t last = g.n_in - 1;
  if constexpr (FROM_F32) {
    const float* row = g.logits + m * g.n_in;
    uint32_t u[P];
#pragma unroll
    for (int p = 0; p < P; ++p) u[p] = __float_as_uint(row[min(i0 + p * STRIDE, last)]);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t i = i0 + p * STRIDE;
      key[p] = i <= last ? ((uint64_t)ord_f32(u[p]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i)
                         : 0ull;
    }
  } else {
    const uint64_t* row = g.keys + m * g.n_in;
#pragma unroll
    for (int p = 0; p < P; ++p) key[p] = row[min(i0 + p * STRIDE, last)];
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (i0 + p * STRIDE > last) key[p] = 0;
  }
}

constexpr int kWaveKeys = 512;  // keys per wave in the k <= 64 path
constexpr int kWavePathMaxK = 64;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <bool FROM_F32>
__global__ void __launch_bounds__(kTopkThreads) k_topk_wave(TopkLevelArgs g) {
  __shared__ uint64_t sel_all[kTopkThreads / 64][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t wc = (int64_t)blockIdx.x * (kTopkThreads / 64) + wv;  // chunk of this wave
  if (wc >= g.chunks) return;  // (no barriers below)
  const int64_t m = blockIdx.y;
  const int64_t base = wc * kWaveKeys;

  uint64_t key[kWaveKeys / 64];
  load_keys<FROM_F32, kWaveKeys / 64, 64>(g, m, base + lane, key);

  uint32_t total = 0;
#pragma unroll
  for (int p = 0; p < kWaveKeys / 64; ++p) total += __popcll(__ballot(key[p] != 0));
  const uint32_t need = total < (uint32_t)g.k ? total : (uint32_t)g.k;
  // Largest T with at least `need` keys >= T (all keys are unique, so then
  // exactly `need`); empty keys (0) are below every trial value.
  uint64_t thresh = 1;
  if (need < total) {
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t trial = T | (1ull << bit);
      uint32_t c = 0;
#pragma unroll
      for (int p = 0; p < kWaveKeys / 64; ++p) c += __popcll(__ballot(key[p] >= trial));
      if (c >= need) {
        T = trial;
        if (c == need) break;
      }
    }
    thresh = T;
  }

  // Compact the `need` selected keys into this wave's LDS row (ds operations
  // of one wave complete in order, so the reads below see these writes).
  uint64_t* sel = sel_all[wv];
  uint32_t off = 0;
#pragma unroll
  for (int p = 0; p < kWaveKeys / 64; ++p) {
    const bool s = key[p] != 0 && key[p] >= thresh;
    const uint64_t b = __ballot(s);
    if (s) sel[off + lanes_below(b)] = key[p];
    off += __popcll(b);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if (g.chunks > 1) {  // candidates for the next level, unsorted, 0-padded to k
    if (lane < g.k) g.keys_out[(m * g.chunks + wc) * g.k + lane] = lane < (int)need ? sel[lane] : 0;
    return;
  }
  if (lane < (int)need) {
    const uint64_t mine = sel[lane];
    int rank = 0;
    for (int j = 0; j < (int)need; ++j) rank += sel[j] > mine ? 1 : 0;
    const uint32_t col = 0xFFFFFFFFu - (uint32_t)mine;
    g.values[m * g.k + rank] = __uint_as_float(unord_f32((uint32_t)(mine >> 32)));
    g.ids[m * g.k + rank] =
        (int64_t)col >= g.n_cols ? -1 : (g.ids_map ? g.ids_map[col] : (int32_t)col);
  }
}

template <bool FROM_F32>
__global__ void __launch_bounds__(kTopkThreads) k_topk_block(TopkLevelArgs g) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sel[kTopkMaxK];
  __shared__ uint32_t s_bin, s_above, s_cnt, s_total, s_nsel;

  const int t = threadIdx.x;
  const int c = blockIdx.x;
  const int64_t m = blockIdx.y;
  const int64_t base = (int64_t)c * kTopkChunk;

  uint64_t key[kTopkPer];
  load_keys<FROM_F32, kTopkPer, kTopkThreads>(g, m, base + t, key);

  // Radix select: find the threshold T with exactly `need` keys >= T.
  uint64_t prefix = 0;  // selected high digits, in place
  uint32_t rem = 0;     // keys still needed inside the current prefix
  uint32_t need = 0;
  uint64_t thresh = 1;  // default: every non-empty key
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    hist[t] = 0;
    if (t == 0) s_nsel = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTopkPer; ++p)
      if (key[p] != 0 && (key[p] & hi_mask) == prefix)
        atomicAdd(&hist[(uint32_t)(key[p] >> shift) & 255u], 1u);
    __syncthreads();
    if (t < 64) {
      // lane l holds bins 255-4l .. 252-4l (descending); inclusive scan over lanes
      uint32_t b4[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) s += (b4[j] = hist[255 - 4 * t - j]);
      uint32_t incl = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, 64);
        if (t >= d) incl += o;
      }
      const uint32_t total = __shfl(incl, 63, 64);
      const uint32_t r = pass == 0 ? (total < (uint32_t)g.k ? total : (uint32_t)g.k) : rem;
      const uint32_t excl = incl - s;
      if (r > 0 && excl < r && r <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + b4[j] >= r) {
            s_bin = 255 - 4 * t - j;
            s_above = cum;
            s_cnt = b4[j];
            break;
          }
          cum += b4[j];
        }
      }
      if (t == 0) s_total = total;
    }
    __syncthreads();
    if (pass == 0) {
      need = s_total < (uint32_t)g.k ? s_total : (uint32_t)g.k;
      rem = need;
      if (need == 0 || need == s_total) break;  // every non-empty key is selected
    }
    rem -= s_above;
    prefix |= (uint64_t)s_bin << shift;
    if (s_cnt == rem) {  // the whole bin is needed: T = prefix, lower digits 0
      thresh = prefix;
      break;
    }
  }

  // Gather the `need` keys >= thresh (unique keys: exactly `need` of them).
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p)
    if (key[p] != 0 && key[p] >= thresh) {
      const uint32_t slot = atomicAdd(&s_nsel, 1u);
      if (slot < (uint32_t)kTopkMaxK) sel[slot] = key[p];
    }
  __syncthreads();

  // Sort by rank: the number of selected keys larger than one's own.
  const bool last = g.chunks == 1;
  for (int i = t; i < g.k; i += kTopkThreads) {
    if (i < (int)need) {
      const uint64_t mine = sel[i];
      int rank = 0;
      for (int j = 0; j < (int)need; ++j) rank += sel[j] > mine ? 1 : 0;
      if (last) {
        const uint32_t col = 0xFFFFFFFFu - (uint32_t)mine;
        g.values[m * g.k + rank] = __uint_as_float(unord_f32((uint32_t)(mine >> 32)));
        // (col < n_cols for every selected key; the check keeps a broken
        // selection from reading outside ids_map)
        g.ids[m * g.k + rank] =
            (int64_t)col >= g.n_cols ? -1 : (g.ids_map ? g.ids_map[col] : (int32_t)col);
      } else {
        g.keys_out[(m * g.chunks + c) * g.k + rank] = mine;
      }
    } else if (!last) {
      g.keys_out[(m * g.chunks + c) * g.k + i] = 0;
    }
  }
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Keys per chunk of one level: a wave's 512 for k <= 64, a workgroup's 2048 above.
inline int64_t chunk_keys(int64_t k) { return k <= kWavePathMaxK ? kWaveKeys : kTopkChunk; }

}  // namespace

size_t topk_workspace_bytes(int64_t M, int64_t n, int64_t k) {
  const int64_t ck = chunk_keys(k);
  const int64_t c1 = ceil_div(n, ck);
  if (c1 <= 1) return 0;
  const int64_t c2 = ceil_div(c1 * k, ck);
  const size_t a = (size_t)(M * c1 * k) * sizeof(uint64_t);
  const size_t b = c2 > 1 ? (size_t)(M * c2 * k) * sizeof(uint64_t) : 0;
  return ((a + 255) / 256) * 256 + b;
}

int launch_topk(const float* logits, int64_t M, int64_t n, int64_t k, const int32_t* ids_map,
                float* values, int32_t* ids, void* workspace, hipStream_t stream) {
  if (k < 1 || k > kTopkMaxK || k > n || M > 65535) return -1;
  const bool wave = k <= kWavePathMaxK;
  const int64_t ck = chunk_keys(k);
  const int64_t c1 = ceil_div(n, ck);
  uint64_t* buf[2] = {static_cast<uint64_t*>(workspace), nullptr};
  if (c1 > 1) {
    if (!workspace) return -1;
    const size_t a = (size_t)(M * c1 * k) * sizeof(uint64_t);
    buf[1] = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + ((a + 255) / 256) * 256);
  }
  // Later levels ping-pong between the two buffers: level i >= 3 writes
  // ceil(.) * k keys per row, never more than level i - 2 wrote there.
  TopkLevelArgs g{};
  g.logits = logits;
  g.n_in = n;
  g.k = (int)k;
  g.values = values;
  g.ids = ids;
  g.ids_map = ids_map;
  g.n_cols = n;
  int cur = 0;
  bool first = true;
  while (true) {
    g.chunks = (int)ceil_div(g.n_in, ck);
    g.keys_out = g.chunks > 1 ? buf[cur] : nullptr;
    const int per_wg = wave ? kTopkThreads / 64 : 1;
    const dim3 grid((unsigned)ceil_div(g.chunks, per_wg), (unsigned)M);
    if (wave) {
      if (first)
        hipLaunchKernelGGL(k_topk_wave<true>, grid, dim3(kTopkThreads), 0, stream, g);
      else
        hipLaunchKernelGGL(k_topk_wave<false>, grid, dim3(kTopkThreads), 0, stream, g);
    } else {
      if (first)
        hipLaunchKernelGGL(k_topk_block<true>, grid, dim3(kTopkThreads), 0, stream, g);
      else
        hipLaunchKernelGGL(k_topk_block<false>, grid, dim3(kTopkThreads), 0, stream, g);
    }
    if (hipGetLastError() != hipSuccess) return -1;
    if (g.chunks == 1) break;
    g.logits = nullptr;
    g.keys = buf[cur];
    g.n_in = (int64_t)g.chunks * k;
    cur ^= 1;
    first = false;
  }
  return 0;
}

}  // namespace nvfp4
