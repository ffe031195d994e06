// gemv.hip -- decode-shaped NVFP4 linear layer (small M) for gfx950.
//
// y[m][j] = sum_k x[m][k] * w[n_j][k], w = e2m1(code) * e4m3(scale) (NVFP4:
// "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding head",
// section "What the artifact is"; W4A16: "What 350+ Experiments Taught Us
// About Serving Qwen 3.6 35B-A3B", section 1).  With row_idx only the listed
// weight rows are read ("The masked head trick" on the first page).
//
// The weights are read exactly once, so the kernel is bound by HBM.  Design:
//  * A wave owns TR tiles of 16 weight rows and a contiguous range of
//    256-element K steps.  The NW waves of a workgroup take different K ranges
//    of the same rows (split-K inside the workgroup); gridDim.y splits K
//    further across workgroups when the row count alone cannot fill the chip.
//  * Per step a lane (n = lane % 16, q = lane / 16) loads two 16-byte words of
//    codes of row n: bytes [16q, 16q+16) and [64+16q, 80+16q) of the step, i.e.
//    elements [32q, 32q+32) and [128+32q, 160+32q).  A wave's load covers 16
//    rows x 64 contiguous bytes -- coalesced 128-bit loads.
//  * Each 32-bit code word (8 elements, one scale) is decoded exactly to bf16
//    in registers and becomes the B operand of one v_mfma_f32_16x16x32_bf16
//    (B[k][n]: lane holds k = 8*(lane/16) .. +7 of column lane%16).  The
//    A operand holds the matching 8 activations of row m = lane % 16, so the
//    32 "k slots" of an MFMA map to scattered physical k -- any bijection works
//    for a dot product as long as A and B agree.
//  * M > 16 uses a second 16-row MFMA tile on the same B operand.
//  * Partial sums are reduced across the NW waves through LDS in wave order,
//    and across workgroups (if gridDim.y > 1) by k_splitk_reduce in split
//    order: results are bit-identical from run to run.
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
  int steps;               // ceil(K / kGemvStep)
  int out_f32;
};

template <int MT, int TR>
__global__ void __launch_bounds__(256) k_gemv(GemvArgs a) {
  extern __shared__ float red[];  // [nw][64][4]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int ln = lane & 15;
  const int64_t K = a.K;

  // K range of this wave: part g of G = gridDim.y * nw equal parts.
  const int G = gridDim.y * nw;
  const int g = blockIdx.y * nw + wave;
  const int s0 = (int)(((int64_t)a.steps * g) / G);
  const int s1 = (int)(((int64_t)a.steps * (g + 1)) / G);

  const uint8_t* cptr[TR];
  const uint8_t* sptr[TR];
  bool rvalid[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int64_t j = ((int64_t)blockIdx.x * TR + t) * 16 + ln;
    rvalid[t] = j < a.n_out;
    const int64_t row = rvalid[t] ? (a.row_idx ? (int64_t)a.row_idx[j] : j) : 0;
    cptr[t] = a.wc + row * (K / 2);
    sptr[t] = a.ws + row * (K / 16);
  }
  const uint16_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + ln;
    xrow[mt] = m < a.M ? a.x + (int64_t)m * K : nullptr;
  }

  f32x4 acc[TR][MT];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemv_accumulate<MT, TR>(acc, xrow, cptr, sptr, rvalid, K, s0, s1);

  // Reduce over the waves (fixed order), then store.
  const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < TR; ++t) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float v = wave_sum_f32x4(red, acc[t][mt]);
      if (threadIdx.x < 256) {
        const int m = mt * 16 + 4 * (l >> 4) + r;
        const int64_t j = ((int64_t)blockIdx.x * TR + t) * 16 + (l & 15);
        if (m < a.M && j < a.n_out) {
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
}

__global__ void __launch_bounds__(256) k_splitk_reduce(const float* __restrict__ partial,
                                                       int splits, int64_t count, int out_f32,
                                                       void* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float v = 0.f;
  for (int z = 0; z < splits; ++z) v += partial[(int64_t)z * count + i];
  if (out_f32)
    static_cast<float*>(out)[i] = v;
  else
    static_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v);
}

template <int MT, int TR>
void launch_gemv_t(const GemvArgs& a, int nw, int zsplit, hipStream_t stream) {
  const int64_t tiles = (a.n_out + 15) / 16;
  dim3 grid((unsigned)((tiles + TR - 1) / TR), (unsigned)zsplit);
  hipLaunchKernelGGL((k_gemv<MT, TR>), grid, dim3(64 * nw), nw * 64 * 4 * sizeof(float), stream,
                     a);
}

}  // namespace

GemvPlan plan_gemv(int64_t M, int64_t n_out, int64_t K, int num_cus) {
  GemvPlan p;
  p.mt = M <= 16 ? 1 : 2;
  p.tr = M <= 16 ? 2 : 4;
  p.nw = 4;
  const int64_t steps = (K + kGemvStep - 1) / kGemvStep;
  const int64_t tiles = (n_out + 15) / 16;
  const int64_t wgs = (tiles + p.tr - 1) / p.tr;
  const int64_t want_waves = (int64_t)num_cus * 8;
  int64_t z = (want_waves + wgs * p.nw - 1) / (wgs * p.nw);
  int64_t zmax = steps / p.nw;  // keep >= 1 step per wave
  if (z > zmax) z = zmax;
  if (z < 1) z = 1;
  p.z = (int)z;
  return p;
}

size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t n_out) {
  return p.z > 1 ? (size_t)p.z * (size_t)M * (size_t)n_out * sizeof(float) : 0;
}

int launch_gemv(const GemvPlan& p, const uint16_t* x, int64_t M, int64_t K, const uint8_t* wc,
                const uint8_t* ws, const int32_t* row_idx, int64_t n_out, bool out_f32,
                void* out, void* workspace, hipStream_t stream) {
  GemvArgs a;
  a.x = x;
  a.wc = wc;
  a.ws = ws;
  a.row_idx = row_idx;
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.K = K;
  a.n_out = n_out;
  a.M = (int)M;
  a.steps = (int)((K + kGemvStep - 1) / kGemvStep);
  a.out_f32 = out_f32 ? 1 : 0;
  if (p.mt == 1 && p.tr == 2)
    launch_gemv_t<1, 2>(a, p.nw, p.z, stream);
  else if (p.mt == 1 && p.tr == 1)
    launch_gemv_t<1, 1>(a, p.nw, p.z, stream);
  else if (p.mt == 1 && p.tr == 4)
    launch_gemv_t<1, 4>(a, p.nw, p.z, stream);
  else if (p.mt == 2 && p.tr == 4)
    launch_gemv_t<2, 4>(a, p.nw, p.z, stream);
  else if (p.mt == 2 && p.tr == 2)
    launch_gemv_t<2, 2>(a, p.nw, p.z, stream);
  else if (p.mt == 2 && p.tr == 1)
    launch_gemv_t<2, 1>(a, p.nw, p.z, stream);
  else
    return -2;
  if (hipGetLastError() != hipSuccess) return -1;
  if (p.z > 1) {
    const int64_t count = M * n_out;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float*>(workspace), p.z, count,
                       out_f32 ? 1 : 0, out);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace nvfp4
