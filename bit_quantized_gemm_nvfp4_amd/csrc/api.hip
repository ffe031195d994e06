// api.hip -- the C ABI of the NVFP4 linear layer (declared in include/nvfp4.h).
//
// Every entry point validates its arguments on the host before it makes any
// HIP call, picks a kernel plan as a pure function of the shape, and enqueues
// on the caller's stream.  The library allocates nothing and keeps no state.
#include <stdlib.h>
#include <stdio.h>

#include <mutex>

#include "../../include/nvfp4.h"
#include "../../include/nvfp4_plan.h"
#include "launch.h"
#include "moe.h"

using namespace nvfp4;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launched(int rc) { return rc == 0 ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH; }

bool log_enabled() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("NVFP4_LOG");
    on = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

// Rows of M handled by one GEMV launch; larger M loops over chunks of this size.
constexpr int64_t kGemvMaxM = 32;
// From this many activation rows on, the MFMA GEMM (weights read once per
// 256-row tile) replaces the weight-streaming GEMV (weights read once per
// 32-row chunk).
constexpr int64_t kGemmMinM = 65;

// Largest K of the MFMA GEMM: its activation offsets inside a 256-row tile are
// 32-bit byte offsets.
constexpr int64_t kGemmMaxK = (int64_t)1 << 22;

struct GemmPlan {
  bool mfma;             // large-M MFMA GEMM
  GemvPlan gemv;
  int64_t m_chunk;       // activation rows per GEMV launch
  size_t a_dequant_bytes;  // W4A4: bf16 copy of the dequantized activations
  size_t partial_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t n_out, bool w4a4,
                   const PlanOverride& ov) {
  (void)N;
  GemmPlan g;
  const int64_t min_m = ov.gemm_min_m >= 1 ? ov.gemm_min_m : kGemmMinM;
  g.mfma = M >= min_m;
  g.m_chunk = M < kGemvMaxM ? M : kGemvMaxM;
  g.gemv = plan_gemv(g.m_chunk, n_out, K, kNumCUs, ov);
  g.partial_bytes = g.mfma ? gemm_workspace_bytes(M, n_out, K, kNumCUs)
                           : gemv_workspace_bytes(g.gemv, g.m_chunk, n_out);
  // W4A4 (NVFP4 activations): the activations are dequantized once (exact in
  // bf16) and the bf16-activation kernels run on them
  g.a_dequant_bytes = w4a4 ? (size_t)M * (size_t)K * 2 : 0;
  return g;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The caller's plan as the internal override; false if it names a layout the
// library does not build (then nothing is launched).
bool to_override(const nvfp4_plan_t* plan, PlanOverride& ov) {
  ov = PlanOverride{};
  if (!plan) return true;
  ov.gemm_min_m = plan->gemm_min_m;
  ov.gemv_small_max = plan->gemv_small_max;
  ov.gemv_tiles = plan->gemv_tiles;
  ov.gemv_waves = plan->gemv_waves;
  ov.gemv_lds_kib = plan->gemv_lds_kib;
  ov.gemv_splits = plan->gemv_splits;
  ov.w4a4_fuse = plan->w4a4_fuse;
  ov.grouped_mfma_min_rows = plan->grouped_mfma_min_rows;
  ov.gemv_kparts = plan->gemv_kparts;
  ov.grouped_gemv_waves = plan->grouped_gemv_waves;
  if (ov.gemm_min_m == 0 || ov.w4a4_fuse > 1) return false;
  if (ov.grouped_gemv_waves >= 0 && ov.grouped_gemv_waves != 4 && ov.grouped_gemv_waves != 8 &&
      ov.grouped_gemv_waves != 16)
    return false;
  return true;
}

// Whether the GEMV layout of a plan exists for activation chunks of M rows
// (the fused W4A4 staging is built for 1 or 2 tiles per wave).
bool gemv_plan_ok(const PlanOverride& ov, int64_t M, int64_t K, bool fused) {
  if (K <= 0 || K % 32 != 0) return true;  // (the entry point reports the shape)
  if (!gemv_override_valid(M, K, ov)) return false;
  if (fused) {
    const GemvPlan p = plan_gemv(M, 1, K, kNumCUs, ov);
    if (p.tr > 2 || ov.gemv_kparts > 1) return false;
  }
  return true;
}

// Whether a plan's GEMV fields name a built tiled layout: the 16x16 kernel
// with 1, 2 or 4 (one activation tile) tiles per wave and 4, 8 or 16 (two
// activation tiles) waves; no K parts inside a workgroup.
bool tiled_plan_ok(const PlanOverride& ov, int64_t M, int64_t K) {
  if (ov.gemv_small_max > 8) return false;
  if (ov.gemv_lds_kib >= 0 && (ov.gemv_lds_kib < 8 || ov.gemv_lds_kib > 160)) return false;
  const GemvPlan p = plan_gemv(M, 1, K, kNumCUs, ov, true);
  if (p.small) {
    if (p.kp > 1)  // one tile per wave, one m-group, 2..16 parts, nw = groups x parts
      return p.mt == 1 && p.tr == 1 && (p.kp == 2 || p.kp == 4 || p.kp == 8 || p.kp == 16) &&
             p.nw % p.kp == 0 && p.nw <= 16 && K / kTileStep >= p.kp;
    return (p.tr == 1 || (p.tr == 2 && p.mt == 1)) && p.nw >= 1 && p.nw <= 8;
  }
  if (p.kp > 1) {  // the built K-parts layouts (as nvfp4_gemm's)
    if ((K + kTileStep - 1) / kTileStep < p.kp) return false;
    if (p.mt == 2) return p.tr == 1 && p.nw == 16 && p.kp == 2;
    if (p.kp == 8 && M > 8) return false;
    static const int lay[][3] = {{2, 2, 4}, {2, 4, 2}, {1, 4, 4}, {1, 4, 2}, {2, 2, 8}, {1, 2, 8},
                                 {2, 1, 8}};
    for (const auto& l : lay)
      if (l[0] == p.tr && l[1] * l[2] == p.nw && l[2] == p.kp) return true;
    return false;
  }
  const bool tr_ok = p.tr == 1 || p.tr == 2 || (p.tr == 4 && p.mt == 1);
  const bool nw_ok = p.nw == 4 || p.nw == 8 || (p.nw == 16 && p.mt == 2);
  return tr_ok && nw_ok;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_SUCCESS: return "NVFP4_SUCCESS";
    case NVFP4_ERROR_INVALID_VALUE: return "NVFP4_ERROR_INVALID_VALUE: null pointer, bad size or misaligned array";
    case NVFP4_ERROR_NOT_SUPPORTED: return "NVFP4_ERROR_NOT_SUPPORTED: shape or dtype not supported";
    case NVFP4_ERROR_WORKSPACE: return "NVFP4_ERROR_WORKSPACE: workspace missing or too small";
    case NVFP4_ERROR_LAUNCH: return "NVFP4_ERROR_LAUNCH: kernel launch failed";
    default: return "NVFP4 unknown status";
  }
}

int nvfp4_version(void) { return 100; }

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                     uint16_t* out, void* stream) {
  if (!codes || !scales || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (N <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out)) return NVFP4_ERROR_INVALID_VALUE;
  if (N * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_dequantize(codes, scales, N, K, out, as_stream(stream)));
}

int nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  if (!x || !codes || !scales) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return NVFP4_ERROR_INVALID_VALUE;
  if (M * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_quantize(x, M, K, codes, scales, as_stream(stream)));
}

size_t nvfp4_gemm_workspace_size(int a_dtype, int64_t M, int64_t N, int64_t K, int64_t n_out) {
  return nvfp4_gemm_workspace_size_planned(nullptr, a_dtype, M, N, K, n_out);
}

void nvfp4_plan_default(nvfp4_plan_t* plan) {
  if (!plan) return;
  plan->gemm_min_m = plan->gemv_small_max = plan->gemv_tiles = plan->gemv_waves = -1;
  plan->gemv_lds_kib = plan->gemv_splits = plan->w4a4_fuse = plan->grouped_mfma_min_rows = -1;
  plan->gemv_kparts = plan->grouped_gemv_waves = -1;
}

size_t nvfp4_gemm_workspace_size_planned(const nvfp4_plan_t* plan, int a_dtype, int64_t M,
                                         int64_t N, int64_t K, int64_t n_out) {
  if (M <= 0 || N <= 0 || K <= 0 || n_out <= 0) return 0;
  PlanOverride ov;
  if (!to_override(plan, ov)) return 0;
  GemmPlan g = plan_gemm(M, N, K, n_out, a_dtype == NVFP4_NVFP4, ov);
  return round_up(g.a_dequant_bytes, 256) + g.partial_bytes;
}

}  // extern "C"

namespace {

// Host checks of the arguments every linear-layer entry point shares (the
// activation operand aside); the status to return, before any launch.
int linear_args_status(const void* a, int64_t M, int64_t N, int64_t K,
                       const uint8_t* w_codes, const uint8_t* w_scales,
                       const int32_t* row_idx, int64_t n_out, int out_dtype, const void* out) {
  if (!a || !w_codes || !w_scales || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || N <= 0 || K <= 0 || n_out <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_FP32) return NVFP4_ERROR_NOT_SUPPORTED;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (row_idx ? n_out > N : n_out != N) return NVFP4_ERROR_INVALID_VALUE;
  if (n_out > INT32_MAX || N > INT32_MAX || M > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(a) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(out) ||
      (row_idx && !aligned16(row_idx)))
    return NVFP4_ERROR_INVALID_VALUE;
  return NVFP4_SUCCESS;
}

int gemm_impl(int a_dtype, const void* a, const uint8_t* a_scales, int64_t M, int64_t N,
              int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
              const int32_t* row_idx, int64_t n_out, int out_dtype, void* out,
              void* workspace, size_t workspace_bytes, void* stream, Alpha alpha,
              const PlanOverride& ov, bool fakequant = false) {
  if (a_dtype != NVFP4_BF16 && a_dtype != NVFP4_NVFP4) return NVFP4_ERROR_NOT_SUPPORTED;
  if (const int rc = linear_args_status(a, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                                        out))
    return rc;
  if (a_dtype == NVFP4_BF16 && a_scales) return NVFP4_ERROR_INVALID_VALUE;
  if (a_dtype == NVFP4_NVFP4 && !a_scales) return NVFP4_ERROR_INVALID_VALUE;
  if (a_scales && !aligned16(a_scales)) return NVFP4_ERROR_INVALID_VALUE;
  const bool w4a4 = a_dtype == NVFP4_NVFP4;
  GemmPlan g = plan_gemm(M, N, K, n_out, w4a4, ov);
  if (g.mfma && K > kGemmMaxK) return NVFP4_ERROR_NOT_SUPPORTED;
  const size_t a_off = 0, p_off = round_up(g.a_dequant_bytes, 256);
  const size_t need = p_off + g.partial_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_ERROR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;

  hipStream_t st = as_stream(stream);
  if (g.mfma) {
    if (((M + 255) / 256) * ((n_out + 255) / 256) > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
    if (log_enabled())
      fprintf(stderr, "[nvfp4] gemm M=%lld N=%lld K=%lld n_out=%lld %s: mfma 256x256\n",
              (long long)M, (long long)N, (long long)K, (long long)n_out, w4a4 ? "w4a4" : "w4a16");
    void* partial = g.partial_bytes ? static_cast<char*>(workspace) + p_off : nullptr;
    const void* xa = a;
    if (w4a4) {
      uint16_t* xd = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + a_off);
      if (launch_dequantize(static_cast<const uint8_t*>(a), a_scales, M, K, xd, st) != 0)
        return NVFP4_ERROR_LAUNCH;
      xa = xd;
    }
    return launched(launch_gemm(fakequant ? GemmA::kFakeQuant : GemmA::kBf16, xa, M, K,
                                w_codes, w_scales, row_idx, n_out,
                                out_dtype == NVFP4_FP32, out, partial, st, alpha));
  }
  const uint16_t* x = static_cast<const uint16_t*>(a);
  if (w4a4) {
    uint16_t* xa = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + a_off);
    if (launch_dequantize(static_cast<const uint8_t*>(a), a_scales, M, K, xa, st) != 0)
      return NVFP4_ERROR_LAUNCH;
    x = xa;
  }
  void* partial = g.partial_bytes ? static_cast<char*>(workspace) + p_off : nullptr;
  const size_t osz = out_dtype == NVFP4_FP32 ? 4 : 2;
  if (log_enabled())
    fprintf(stderr, "[nvfp4] gemm M=%lld N=%lld K=%lld n_out=%lld %s: gemv%s mt=%d tr=%d nw=%d z=%d m_chunk=%lld\n",
            (long long)M, (long long)N, (long long)K, (long long)n_out, w4a4 ? "w4a4" : "w4a16",
            g.gemv.small ? "4x4x4" : "16x16x32", g.gemv.mt, g.gemv.tr, g.gemv.nw, g.gemv.z,
            (long long)g.m_chunk);
  for (int64_t m0 = 0; m0 < M; m0 += g.m_chunk) {
    const int64_t mc = (M - m0) < g.m_chunk ? (M - m0) : g.m_chunk;
    int rc = launch_gemv(g.gemv, x + m0 * K, mc, K, w_codes, w_scales, row_idx, n_out,
                         out_dtype == NVFP4_FP32, static_cast<char*>(out) + m0 * n_out * osz,
                         partial, st, alpha, fakequant);
    if (rc != 0) return NVFP4_ERROR_LAUNCH;
  }
  return NVFP4_SUCCESS;
}

}  // namespace

extern "C" {

int nvfp4_gemm(int a_dtype, const void* a, const uint8_t* a_scales, int64_t M, int64_t N,
               int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
               const int32_t* row_idx, int64_t n_out, int out_dtype, void* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(a_dtype, a, a_scales, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                   out, workspace, workspace_bytes, stream, Alpha{}, PlanOverride{});
}

int nvfp4_gemm_planned(const nvfp4_plan_t* plan, int a_dtype, const void* a,
                       const uint8_t* a_scales, int64_t M, int64_t N, int64_t K,
                       const uint8_t* w_codes, const uint8_t* w_scales, const int32_t* row_idx,
                       int64_t n_out, int out_dtype, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  if (M > 0 && !gemv_plan_ok(ov, M < 32 ? M : 32, K, false)) return NVFP4_ERROR_INVALID_VALUE;
  return gemm_impl(a_dtype, a, a_scales, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                   out, workspace, workspace_bytes, stream, Alpha{}, ov);
}

int nvfp4_gemm_scaled(int a_dtype, const void* a, const uint8_t* a_scales,
                      const float* a_global_scale, int64_t M, int64_t N, int64_t K,
                      const uint8_t* w_codes, const uint8_t* w_scales,
                      const float* w_global_scale, const int32_t* row_idx, int64_t n_out,
                      int out_dtype, void* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (a_dtype != NVFP4_NVFP4 && a_global_scale) return NVFP4_ERROR_INVALID_VALUE;
  if ((a_global_scale && (reinterpret_cast<uintptr_t>(a_global_scale) & 3u)) ||
      (w_global_scale && (reinterpret_cast<uintptr_t>(w_global_scale) & 3u)))
    return NVFP4_ERROR_INVALID_VALUE;
  Alpha alpha;
  alpha.a = a_global_scale;
  alpha.w = w_global_scale;
  return gemm_impl(a_dtype, a, a_scales, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                   out, workspace, workspace_bytes, stream, alpha, PlanOverride{});
}

// ---- tiled weights --------------------------------------------------------------

namespace {

struct TiledPlan {
  bool mfma;  // large M: the MFMA GEMM reading tiled weights
  GemvPlan gemv;
  int64_t m_chunk;
  size_t a_dequant_bytes;
  size_t partial_bytes;
};

TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K, bool w4a4, const PlanOverride& ov) {
  TiledPlan t;
  const int64_t min_m = ov.gemm_min_m >= 1 ? ov.gemm_min_m : kGemmMinM;
  t.mfma = M >= min_m;
  t.m_chunk = M < kGemvMaxM ? M : kGemvMaxM;
  t.gemv = plan_gemv(t.m_chunk, N, K, kNumCUs, ov, true);
  t.partial_bytes = t.mfma ? gemm_workspace_bytes(M, N, K, kNumCUs)
                           : gemv_workspace_bytes(t.gemv, t.m_chunk, N);
  t.a_dequant_bytes = w4a4 ? (size_t)M * (size_t)K * 2 : 0;
  return t;
}

size_t tiled_workspace(int a_dtype, int64_t M, int64_t N, int64_t K, const PlanOverride& ov) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const TiledPlan t = plan_tiled(M, N, K, a_dtype == NVFP4_NVFP4, ov);
  const size_t p_off = round_up(t.a_dequant_bytes, 256);
  return p_off + t.partial_bytes == 0 ? 0 : p_off + t.partial_bytes;
}

int gemm_tiled_impl(int a_dtype, const void* a, const uint8_t* a_scales, int64_t M, int64_t N,
                    int64_t K, const uint8_t* w_tiled, int out_dtype, void* out, void* workspace,
                    size_t workspace_bytes, void* stream, const PlanOverride& ov) {
  if (a_dtype != NVFP4_BF16 && a_dtype != NVFP4_NVFP4) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!a || !w_tiled || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || N <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_FP32) return NVFP4_ERROR_NOT_SUPPORTED;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (N > INT32_MAX || M > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
  if (N * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(a) || !aligned16(w_tiled) || !aligned16(out)) return NVFP4_ERROR_INVALID_VALUE;
  if ((a_dtype == NVFP4_BF16) != (a_scales == nullptr)) return NVFP4_ERROR_INVALID_VALUE;
  if (a_scales && !aligned16(a_scales)) return NVFP4_ERROR_INVALID_VALUE;
  const bool w4a4 = a_dtype == NVFP4_NVFP4;
  const TiledPlan t = plan_tiled(M, N, K, w4a4, ov);
  if (t.mfma && K > kGemmMaxK) return NVFP4_ERROR_NOT_SUPPORTED;
  if (t.mfma && ((M + 255) / 256) * ((N + 255) / 256) > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
  const size_t p_off = round_up(t.a_dequant_bytes, 256);
  const size_t need = p_off + t.partial_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_ERROR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  hipStream_t st = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(a);
  if (w4a4) {
    uint16_t* xa = static_cast<uint16_t*>(workspace);
    if (launch_dequantize(static_cast<const uint8_t*>(a), a_scales, M, K, xa, st) != 0)
      return NVFP4_ERROR_LAUNCH;
    x = xa;
  }
  void* partial = t.partial_bytes ? static_cast<char*>(workspace) + p_off : nullptr;
  if (t.mfma)
    return launched(launch_gemm(GemmA::kBf16, x, M, K, w_tiled, nullptr, nullptr, N,
                                out_dtype == NVFP4_FP32, out, partial, st, Alpha{}, true));
  const size_t osz = out_dtype == NVFP4_FP32 ? 4 : 2;
  if (log_enabled())
    fprintf(stderr, "[nvfp4] gemm_tiled M=%lld N=%lld K=%lld: mt=%d tr=%d nw=%d z=%d\n",
            (long long)M, (long long)N, (long long)K, t.gemv.mt, t.gemv.tr, t.gemv.nw, t.gemv.z);
  for (int64_t m0 = 0; m0 < M; m0 += t.m_chunk) {
    const int64_t mc = (M - m0) < t.m_chunk ? (M - m0) : t.m_chunk;
    if (launch_gemv_tiled(t.gemv, x + m0 * K, mc, K, w_tiled, N, out_dtype == NVFP4_FP32,
                          static_cast<char*>(out) + m0 * N * osz, partial, st) != 0)
      return NVFP4_ERROR_LAUNCH;
  }
  return NVFP4_SUCCESS;
}

}  // namespace

extern "C" {

size_t nvfp4_tiled_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 32 != 0) return 0;
  return tiled_weight_bytes(N, K);
}

int nvfp4_tile_weight(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                      const int32_t* row_idx, int64_t n_rows, uint8_t* w_tiled, void* stream) {
  if (!codes || !scales || !w_tiled) return NVFP4_ERROR_INVALID_VALUE;
  if (N <= 0 || K <= 0 || n_rows <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (row_idx ? n_rows > N : n_rows != N) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (N > INT32_MAX || N * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  // one thread per 16-byte piece, in workgroups of 256
  if (tiled_weight_bytes(n_rows, K) / 16 / 256 >= (size_t)INT32_MAX)
    return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(w_tiled) ||
      (row_idx && !aligned16(row_idx)))
    return NVFP4_ERROR_INVALID_VALUE;
  return launched(launch_tile_weight(codes, scales, row_idx, n_rows, K, w_tiled,
                                     as_stream(stream)));
}

size_t nvfp4_gemm_tiled_workspace_size(int a_dtype, int64_t M, int64_t N, int64_t K) {
  return tiled_workspace(a_dtype, M, N, K, PlanOverride{});
}

int nvfp4_gemm_tiled(int a_dtype, const void* a, const uint8_t* a_scales, int64_t M, int64_t N,
                     int64_t K, const uint8_t* w_tiled, int out_dtype, void* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_tiled_impl(a_dtype, a, a_scales, M, N, K, w_tiled, out_dtype, out, workspace,
                         workspace_bytes, stream, PlanOverride{});
}

size_t nvfp4_gemm_tiled_workspace_size_planned(const nvfp4_plan_t* plan, int a_dtype, int64_t M,
                                               int64_t N, int64_t K) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return 0;
  return tiled_workspace(a_dtype, M, N, K, ov);
}

int nvfp4_gemm_tiled_planned(const nvfp4_plan_t* plan, int a_dtype, const void* a,
                             const uint8_t* a_scales, int64_t M, int64_t N, int64_t K,
                             const uint8_t* w_tiled, int out_dtype, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  if (M > 0 && K > 0 && K % 32 == 0 && !tiled_plan_ok(ov, M < 32 ? M : 32, K))
    return NVFP4_ERROR_INVALID_VALUE;
  return gemm_tiled_impl(a_dtype, a, a_scales, M, N, K, w_tiled, out_dtype, out, workspace,
                         workspace_bytes, stream, ov);
}

}  // extern "C"

// W4A4 from bf16 activations.  The kernel can quantize the activations
// itself as it loads them (no extra launch and no activation copy in memory),
// but every workgroup along N then repeats that work; otherwise one pass
// writes the quantized-and-dequantized activations (bf16, exact) and the
// plain bf16-activation kernel reads them.  In the GEMV staging wins only for
// very few rows on narrow layers; in the MFMA GEMM's tile loads it does not
// win (measured: DESIGN notes), so large M takes the pass.
static bool w4a4_fuse(const GemmPlan& g, int64_t M, int64_t n_out, const PlanOverride& ov) {
  if (ov.w4a4_fuse >= 0) return ov.w4a4_fuse == 1;
  return !g.mfma && M <= 4 && n_out <= 65536;
}

static size_t w4a4_bf16_workspace(const PlanOverride& ov, int64_t M, int64_t N, int64_t K,
                                  int64_t n_out) {
  if (M <= 0 || N <= 0 || K <= 0 || n_out <= 0) return 0;
  const GemmPlan g = plan_gemm(M, N, K, n_out, false, ov);
  if (w4a4_fuse(g, M, n_out, ov)) return g.partial_bytes;
  return round_up((size_t)M * (size_t)K * 2, 256) + g.partial_bytes;
}

static int w4a4_bf16_impl(const PlanOverride& ov, const uint16_t* a, int64_t M, int64_t N,
                          int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                          const int32_t* row_idx, int64_t n_out, int out_dtype, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (const int rc = linear_args_status(a, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                                        out))
    return rc;  // (checked here, before the quantizer runs)
  if (M * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  const GemmPlan g = plan_gemm(M, N, K, n_out, false, ov);
  if (g.mfma && K > kGemmMaxK) return NVFP4_ERROR_NOT_SUPPORTED;
  const size_t need = w4a4_bf16_workspace(ov, M, N, K, n_out);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_ERROR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = as_stream(stream);
  if (w4a4_fuse(g, M, n_out, ov))  // quantized inside the kernel's activation loads
    return gemm_impl(NVFP4_BF16, a, nullptr, M, N, K, w_codes, w_scales, row_idx, n_out,
                     out_dtype, out, workspace, workspace_bytes, stream, Alpha{}, ov, true);
  // one pass writes the activations quantized to NVFP4 and dequantized (bf16,
  // exact), then the bf16-activation GEMV or MFMA GEMM runs on them
  uint16_t* xq = reinterpret_cast<uint16_t*>(ws);
  const size_t g_off = round_up((size_t)M * (size_t)K * 2, 256);
  if (launch_fakequant(a, M, K, xq, st) != 0) return NVFP4_ERROR_LAUNCH;
  return gemm_impl(NVFP4_BF16, xq, nullptr, M, N, K, w_codes, w_scales, row_idx, n_out,
                   out_dtype, out, g.partial_bytes ? ws + g_off : nullptr,
                   workspace_bytes - g_off, stream, Alpha{}, ov);
}

size_t nvfp4_gemm_w4a4_bf16_workspace_size(int64_t M, int64_t N, int64_t K, int64_t n_out) {
  return w4a4_bf16_workspace(PlanOverride{}, M, N, K, n_out);
}

int nvfp4_gemm_w4a4_bf16(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         const int32_t* row_idx, int64_t n_out, int out_dtype, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return w4a4_bf16_impl(PlanOverride{}, a, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                        out, workspace, workspace_bytes, stream);
}

size_t nvfp4_gemm_w4a4_bf16_workspace_size_planned(const nvfp4_plan_t* plan, int64_t M,
                                                   int64_t N, int64_t K, int64_t n_out) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return 0;
  return w4a4_bf16_workspace(ov, M, N, K, n_out);
}

int nvfp4_gemm_w4a4_bf16_planned(const nvfp4_plan_t* plan, const uint16_t* a, int64_t M,
                                 int64_t N, int64_t K, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const int32_t* row_idx, int64_t n_out,
                                 int out_dtype, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  if (M > 0 && !gemv_plan_ok(ov, M < 32 ? M : 32, K, ov.w4a4_fuse == 1))
    return NVFP4_ERROR_INVALID_VALUE;
  return w4a4_bf16_impl(ov, a, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype, out,
                        workspace, workspace_bytes, stream);
}

int nvfp4_quantize_scaled(const uint16_t* x, int64_t M, int64_t K, const float* global_scale,
                          uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !global_scale || !codes || !scales) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(global_scale) & 3u))
    return NVFP4_ERROR_INVALID_VALUE;
  if (M * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_quantize_scaled(x, M, K, global_scale, codes, scales, as_stream(stream)));
}

size_t nvfp4_quantize_weight_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return quantize_weight_workspace_bytes();
}

int nvfp4_quantize_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes,
                          uint8_t* scales, float* global_scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!w || !codes || !scales || !global_scale) return NVFP4_ERROR_INVALID_VALUE;
  if (N <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(global_scale) & 3u))
    return NVFP4_ERROR_INVALID_VALUE;
  if (N * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!workspace || workspace_bytes < quantize_weight_workspace_bytes())
    return NVFP4_ERROR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  return launched(launch_quantize_weight(w, N, K, codes, scales, global_scale, workspace,
                                         as_stream(stream)));
}

int nvfp4_dequantize_scaled(const uint8_t* codes, const uint8_t* scales,
                            const float* global_scale, int64_t N, int64_t K, uint16_t* out,
                            void* stream) {
  if (!codes || !scales || !global_scale || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (N <= 0 || K <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(global_scale) & 3u))
    return NVFP4_ERROR_INVALID_VALUE;
  if (N * (K / 32) > ((int64_t)1 << 40)) return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_dequantize_scaled(codes, scales, global_scale, N, K, out,
                                           as_stream(stream)));
}

size_t nvfp4_topk_workspace_size(int64_t M, int64_t n, int64_t k) {
  if (M <= 0 || n <= 0 || k <= 0) return 0;
  return topk_workspace_bytes(M, n, k);
}

int nvfp4_topk(const float* logits, int64_t M, int64_t n, int64_t k, const int32_t* ids_map,
               float* values, int32_t* ids, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (!logits || !values || !ids) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || n <= 0 || k <= 0 || k > n) return NVFP4_ERROR_INVALID_VALUE;
  if (k > kTopkMaxK || n > INT32_MAX || M > 65535) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(logits) || !aligned16(values) || !aligned16(ids) ||
      (ids_map && !aligned16(ids_map)))
    return NVFP4_ERROR_INVALID_VALUE;
  const size_t need = topk_workspace_bytes(M, n, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_ERROR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  return launched(launch_topk(logits, M, n, k, ids_map, values, ids, workspace,
                              as_stream(stream)));
}

size_t nvfp4_head_topk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t n_out,
                                      int64_t k) {
  if (M <= 0 || N <= 0 || K <= 0 || n_out <= 0 || k <= 0) return 0;
  return round_up((size_t)M * (size_t)n_out * sizeof(float), 256) +
         round_up(nvfp4_gemm_workspace_size(NVFP4_BF16, M, N, K, n_out), 256) +
         topk_workspace_bytes(M, n_out, k);
}

int nvfp4_head_topk(const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w_codes,
                    const uint8_t* w_scales, const int32_t* row_idx, int64_t n_out, int64_t k,
                    float* values, int32_t* ids, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!a || !w_codes || !w_scales || !values || !ids) return NVFP4_ERROR_INVALID_VALUE;
  if (M <= 0 || N <= 0 || K <= 0 || n_out <= 0 || k <= 0 || k > n_out)
    return NVFP4_ERROR_INVALID_VALUE;
  if (k > kTopkMaxK || M > 65535) return NVFP4_ERROR_NOT_SUPPORTED;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (row_idx ? n_out > N : n_out != N) return NVFP4_ERROR_INVALID_VALUE;
  if (n_out > INT32_MAX || N > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(a) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(values) ||
      !aligned16(ids) || (row_idx && !aligned16(row_idx)))
    return NVFP4_ERROR_INVALID_VALUE;
  const size_t need = nvfp4_head_topk_workspace_size(M, N, K, n_out, k);
  if (!workspace || workspace_bytes < need) return NVFP4_ERROR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws);
  const size_t g_off = round_up((size_t)M * (size_t)n_out * sizeof(float), 256);
  const size_t g_bytes = nvfp4_gemm_workspace_size(NVFP4_BF16, M, N, K, n_out);
  const size_t t_off = g_off + round_up(g_bytes, 256);
  const int rc = nvfp4_gemm(NVFP4_BF16, a, nullptr, M, N, K, w_codes, w_scales, row_idx, n_out,
                            NVFP4_FP32, logits, g_bytes ? ws + g_off : nullptr, g_bytes, stream);
  if (rc != NVFP4_SUCCESS) return rc;
  const size_t t_bytes = topk_workspace_bytes(M, n_out, k);
  return launched(launch_topk(logits, M, n_out, k, row_idx, values, ids,
                              t_bytes ? ws + t_off : nullptr, as_stream(stream)));
}

int nvfp4_kv_store_e4m3(const uint16_t* x, int64_t T, int64_t W, const int32_t* slot_mapping,
                        float scale, uint8_t* cache, int64_t num_slots, void* stream) {
  if (!x || !slot_mapping || !cache) return NVFP4_ERROR_INVALID_VALUE;
  if (T <= 0 || W <= 0 || num_slots <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (!(scale >= 0x1p-126f && scale <= 3.4028235e38f)) return NVFP4_ERROR_INVALID_VALUE;
  if (W % 16 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(x) || !aligned16(cache)) return NVFP4_ERROR_INVALID_VALUE;
  if (T * W > ((int64_t)1 << 40) || num_slots * W > ((int64_t)1 << 40))
    return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_kv_store(x, T, W, slot_mapping, scale, cache, num_slots,
                                  as_stream(stream)));
}

int nvfp4_kv_load_e4m3(const uint8_t* cache, int64_t num_slots, int64_t W,
                       const int32_t* block_table, const int32_t* seq_lens, int64_t B,
                       int64_t max_pages, int64_t page_size, int64_t max_len, float scale,
                       uint16_t* out, void* stream) {
  if (!cache || !block_table || !seq_lens || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (num_slots <= 0 || W <= 0 || B <= 0 || max_pages <= 0 || page_size <= 0 || max_len <= 0)
    return NVFP4_ERROR_INVALID_VALUE;
  if (!(scale >= 0x1p-126f && scale <= 3.4028235e38f)) return NVFP4_ERROR_INVALID_VALUE;
  if (W % 16 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(cache) || !aligned16(out)) return NVFP4_ERROR_INVALID_VALUE;
  if (B * max_len * W > ((int64_t)1 << 40) || num_slots * W > ((int64_t)1 << 40))
    return NVFP4_ERROR_NOT_SUPPORTED;
  return launched(launch_kv_load(cache, num_slots, W, block_table, seq_lens, B, max_pages,
                                 page_size, max_len, scale, out, as_stream(stream)));
}

size_t nvfp4_moe_align_workspace_size(int64_t T, int64_t topk, int64_t E) {
  if (T <= 0 || topk <= 0 || E <= 0) return 0;
  return moe_align_workspace_bytes(T, topk, E);
}

int nvfp4_moe_align(const int32_t* topk_ids, const float* gates, int64_t T, int64_t topk,
                    int64_t E, int32_t* expert_offsets, int32_t* gather_idx,
                    int32_t* slot_pos, float* row_gates, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!topk_ids || !expert_offsets || !gather_idx || !slot_pos) return NVFP4_ERROR_INVALID_VALUE;
  if ((gates == nullptr) != (row_gates == nullptr)) return NVFP4_ERROR_INVALID_VALUE;
  if ((gates && !aligned16(gates)) || (row_gates && !aligned16(row_gates)))
    return NVFP4_ERROR_INVALID_VALUE;
  if (T <= 0 || topk <= 0 || E <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (topk > 32 || E > kMoeMaxExperts || T * topk > INT32_MAX / 2) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(topk_ids) || !aligned16(expert_offsets) || !aligned16(gather_idx) ||
      !aligned16(slot_pos))
    return NVFP4_ERROR_INVALID_VALUE;
  const size_t need = moe_align_workspace_bytes(T, topk, E);
  if (!workspace || workspace_bytes < need) return NVFP4_ERROR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERROR_INVALID_VALUE;
  return launched(launch_moe_align(topk_ids, gates, T, topk, E, expert_offsets, gather_idx,
                                   slot_pos, row_gates, workspace, as_stream(stream)));
}

size_t nvfp4_grouped_gemm_workspace_size(int64_t R, int64_t E, int64_t N, int64_t K) {
  if (R <= 0 || E <= 0 || N <= 0 || K <= 0) return 0;
  return moe_grouped_workspace_bytes(R, E, N, K);
}

}  // extern "C"

static int grouped_impl(const PlanOverride& ov, const uint16_t* a, int64_t a_rows, int64_t K,
                        const int32_t* gather_idx, const int32_t* expert_offsets, int64_t E,
                        int64_t R, int64_t N, const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* w_global, const float* row_scale, int epilogue,
                        uint16_t* out, void* workspace, size_t workspace_bytes, void* stream,
                        bool tiled = false) {
  if (!a || !expert_offsets || !w_codes || (!tiled && !w_scales) || !out)
    return NVFP4_ERROR_INVALID_VALUE;
  if (w_global && reinterpret_cast<uintptr_t>(w_global) % alignof(float) != 0)
    return NVFP4_ERROR_INVALID_VALUE;
  if (a_rows <= 0 || K <= 0 || E <= 0 || R <= 0 || N <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (K % 32 != 0) return NVFP4_ERROR_NOT_SUPPORTED;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_SWIGLU) return NVFP4_ERROR_NOT_SUPPORTED;
  if (epilogue == NVFP4_EPI_SWIGLU && (N % 32 != 0)) return NVFP4_ERROR_NOT_SUPPORTED;
  if (N % 16 != 0 || E > kMoeMaxExperts || R > INT32_MAX || a_rows > INT32_MAX)
    return NVFP4_ERROR_NOT_SUPPORTED;
  if (!gather_idx && a_rows < R) return NVFP4_ERROR_INVALID_VALUE;
  if (!aligned16(a) || !aligned16(expert_offsets) || !aligned16(w_codes) ||
      (!tiled && !aligned16(w_scales)) || !aligned16(out) ||
      (gather_idx && !aligned16(gather_idx)) || (row_scale && !aligned16(row_scale)))
    return NVFP4_ERROR_INVALID_VALUE;
  if (grouped_path(a_rows, K, E, R, ov) == GroupedPath::kNone) return NVFP4_ERROR_NOT_SUPPORTED;
  const size_t need = moe_grouped_workspace_bytes(R, E, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_ERROR_WORKSPACE;
  return launched(launch_grouped_gemm(a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_codes,
                                      tiled ? nullptr : w_scales, w_global, row_scale,
                                      epilogue == NVFP4_EPI_SWIGLU, out, workspace,
                                      as_stream(stream), ov, tiled));
}

extern "C" {

int nvfp4_grouped_gemm(const uint16_t* a, int64_t a_rows, int64_t K, const int32_t* gather_idx,
                       const int32_t* expert_offsets, int64_t E, int64_t R, int64_t N,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* row_scale,
                       int epilogue, uint16_t* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return grouped_impl(PlanOverride{}, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_codes,
                      w_scales, nullptr, row_scale, epilogue, out, workspace, workspace_bytes,
                      stream);
}

int nvfp4_grouped_gemm_scaled(const uint16_t* a, int64_t a_rows, int64_t K,
                              const int32_t* gather_idx, const int32_t* expert_offsets, int64_t E,
                              int64_t R, int64_t N, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* w_global_scales,
                              const float* row_scale, int epilogue, uint16_t* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_impl(PlanOverride{}, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_codes,
                      w_scales, w_global_scales, row_scale, epilogue, out, workspace,
                      workspace_bytes, stream);
}

int nvfp4_grouped_gemm_planned(const nvfp4_plan_t* plan, const uint16_t* a, int64_t a_rows,
                               int64_t K, const int32_t* gather_idx,
                               const int32_t* expert_offsets, int64_t E, int64_t R, int64_t N,
                               const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* row_scale, int epilogue, uint16_t* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  return grouped_impl(ov, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_codes, w_scales,
                      nullptr, row_scale, epilogue, out, workspace, workspace_bytes, stream);
}

int nvfp4_grouped_gemm_scaled_planned(const nvfp4_plan_t* plan, const uint16_t* a,
                                      int64_t a_rows, int64_t K, const int32_t* gather_idx,
                                      const int32_t* expert_offsets, int64_t E, int64_t R,
                                      int64_t N, const uint8_t* w_codes, const uint8_t* w_scales,
                                      const float* w_global_scales, const float* row_scale,
                                      int epilogue, uint16_t* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  return grouped_impl(ov, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_codes, w_scales,
                      w_global_scales, row_scale, epilogue, out, workspace, workspace_bytes,
                      stream);
}

int nvfp4_grouped_gemm_tiled(const uint16_t* a, int64_t a_rows, int64_t K,
                             const int32_t* gather_idx, const int32_t* expert_offsets, int64_t E,
                             int64_t R, int64_t N, const uint8_t* w_tiled,
                             const float* w_global_scales, const float* row_scale, int epilogue,
                             uint16_t* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return grouped_impl(PlanOverride{}, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_tiled,
                      nullptr, w_global_scales, row_scale, epilogue, out, workspace,
                      workspace_bytes, stream, true);
}

int nvfp4_grouped_gemm_tiled_planned(const nvfp4_plan_t* plan, const uint16_t* a, int64_t a_rows,
                                     int64_t K, const int32_t* gather_idx,
                                     const int32_t* expert_offsets, int64_t E, int64_t R,
                                     int64_t N, const uint8_t* w_tiled,
                                     const float* w_global_scales, const float* row_scale,
                                     int epilogue, uint16_t* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  PlanOverride ov;
  if (!to_override(plan, ov)) return NVFP4_ERROR_INVALID_VALUE;
  return grouped_impl(ov, a, a_rows, K, gather_idx, expert_offsets, E, R, N, w_tiled, nullptr,
                      w_global_scales, row_scale, epilogue, out, workspace, workspace_bytes,
                      stream, true);
}

int nvfp4_moe_combine(const uint16_t* y, const int32_t* slot_pos, int64_t T, int64_t topk,
                      int64_t H, uint16_t* out, void* stream) {
  if (!y || !slot_pos || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (T <= 0 || topk <= 0 || H <= 0) return NVFP4_ERROR_INVALID_VALUE;
  if (H % 8 != 0 || topk > 32 || T * topk > INT32_MAX) return NVFP4_ERROR_NOT_SUPPORTED;
  if (!aligned16(y) || !aligned16(slot_pos) || !aligned16(out)) return NVFP4_ERROR_INVALID_VALUE;
  return launched(launch_moe_combine(y, slot_pos, T, topk, H, out, as_stream(stream)));
}

}  // extern "C"

// ---- the entry point that allocates nothing ---------------------------------------
//
// nvfp4_gemm_noalloc keeps its workspace in `scratch`, a file-scope device
// array: every GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory,
// so its address on each device is looked up once with hipGetSymbolAddress
// (with that device current) and only that address is passed to the kernels.

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

// This device's address of `scratch` (looked up on the first call on the
// device); nullptr if the lookup fails.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t nvfp4_noalloc_scratch_bytes(void) { return kScratchBytes; }

int nvfp4_gemm_noalloc(int a_dtype, const void* a, const uint8_t* a_scales, int64_t M, int64_t N,
                       int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                       const int32_t* row_idx, int64_t n_out, int out_dtype, void* out,
                       void* stream) {
  // the host checks of nvfp4_gemm first, so an invalid call makes no HIP call
  if (a_dtype != NVFP4_BF16 && a_dtype != NVFP4_NVFP4) return NVFP4_ERROR_NOT_SUPPORTED;
  if (const int rc = linear_args_status(a, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                                        out))
    return rc;
  if ((a_dtype == NVFP4_BF16) != (a_scales == nullptr)) return NVFP4_ERROR_INVALID_VALUE;
  if (a_scales && !aligned16(a_scales)) return NVFP4_ERROR_INVALID_VALUE;
  const size_t need = nvfp4_gemm_workspace_size(a_dtype, M, N, K, n_out);
  if (need > kScratchBytes) return NVFP4_ERROR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device();
    if (!ws) return NVFP4_ERROR_LAUNCH;
  }
  return gemm_impl(a_dtype, a, a_scales, M, N, K, w_codes, w_scales, row_idx, n_out, out_dtype,
                   out, ws, need > 0 ? kScratchBytes : 0, stream, Alpha{}, PlanOverride{});
}

}  // extern "C"
