// tile.hip -- the tiled NVFP4 weight layout ("NF4T"): conversion from the
// row-major pair of arrays (codes [N][K/2], scales [N][K/16]), all rows or a
// listed subset of them (a fixed row set such as a masked head's ids).
//
// The elements and their values are those of the row-major matrix (NVFP4 as
// in "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding head",
// section "What the artifact is"); only the byte order changes, once, when the
// weights are loaded.  Rows are grouped in tiles of 16, K in steps of 256
// elements; one (tile, step) block is 2,304 contiguous bytes:
//
//   [   0, 1024)  codes, half 0: lane L's 16 bytes at 16 L
//   [1024, 2048)  codes, half 1: lane L's 16 bytes at 1024 + 16 L
//   [2048, 2304)  scales: lane L's 4 bytes at 2048 + 4 L
//
// where lane L = 16 q + n (n = L % 16, q = L / 16) stands for row 16 t + n and
// the elements [256 s + 64 q, 256 s + 64 q + 64) of that row: half h holds
// the code bytes of elements 256 s + 64 q + 32 h .. + 31 (same nibble order as
// the row-major codes), the four scale bytes those 64 elements use.  Blocks
// run tile-major: block (t, s) starts at byte (t * S + s) * 2304, S = ceil(K /
// 256), so a tile's whole K range is contiguous.  Rows past N and elements
// past K are zero codes with zero scales (value 0).
//
// A wave of the streaming kernels reads one block as three fully used,
// contiguous runs (two 1 KB code loads and one 256 B scale load), and the
// scale bytes arrive in the same stream as the codes.
#include "device.h"
#include "launch.h"

namespace nvfp4 {

namespace {

// One thread per 16-byte piece of the tiled array: pieces 0..127 of a block
// are code pieces (half = p / 64, lane = p % 64), 128..143 scale pieces (four
// lanes each).
// Tiled row r is row-major row row_idx[r] (r when row_idx is null), r < R.
__global__ void __launch_bounds__(256) k_tile_weight(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const int32_t* __restrict__ row_idx,
                                                     int64_t R, int64_t K, int64_t S,
                                                     int64_t pieces, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int64_t blk = i / 144;
  const int p = (int)(i - blk * 144);
  const int64_t t = blk / S, s = blk - t * S;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (p < 128) {
    const int h = p >> 6, lane = p & 63;
    const int64_t r = t * 16 + (lane & 15);
    const int64_t k = s * kTileStep + 64 * (lane >> 4) + 32 * h;  // K % 32 == 0: all or none
    if (r < R && k < K) {
      const int64_t row = row_idx ? (int64_t)row_idx[r] : r;
      v = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k / 2);
    }
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lane = 4 * (p - 128) + j;
      const int64_t r = t * 16 + (lane & 15);
      const int64_t b0 = s * (kTileStep / 16) + 4 * (lane >> 4);  // first scale block
      if (r >= R) continue;
      const int64_t row = row_idx ? (int64_t)row_idx[r] : r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b0 + e < K / 16) w[j] |= (uint32_t)scales[row * (K / 16) + b0 + e] << (8 * e);
    }
    v = u32x4{w[0], w[1], w[2], w[3]};
  }
  *reinterpret_cast<u32x4*>(out + blk * kTileBlockBytes + 16 * p) = v;
}

}  // namespace

size_t tiled_weight_bytes(int64_t N, int64_t K) {
  const int64_t T = (N + kTileRows - 1) / kTileRows, S = (K + kTileStep - 1) / kTileStep;
  return (size_t)T * (size_t)S * kTileBlockBytes;
}

int launch_tile_weight(const uint8_t* codes, const uint8_t* scales, const int32_t* row_idx,
                       int64_t R, int64_t K, uint8_t* out, hipStream_t stream) {
  const int64_t T = (R + kTileRows - 1) / kTileRows, S = (K + kTileStep - 1) / kTileStep;
  const int64_t pieces = T * S * (kTileBlockBytes / 16);
  const int64_t blocks = (pieces + 255) / 256;
  if (blocks > INT32_MAX) return -2;
  hipLaunchKernelGGL(k_tile_weight, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales,
                     row_idx, R, K, S, pieces, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
