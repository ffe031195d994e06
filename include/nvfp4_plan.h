/*
 * nvfp4_plan.h -- launch-plan overrides of the NVFP4 linear layer, for tests
 * and tuning sweeps.
 *
 * The entry points of nvfp4.h choose their kernels and launch shapes as a pure
 * function of the problem shape.  The *_planned variants below compute the same
 * results (same operation, arguments, layouts, tolerances and determinism as the
 * entry point they extend) with parts of that choice made by the caller, so that
 * every kernel layout can be driven at sizes an oracle checks whole, and a sweep
 * can time the alternatives.  They keep no state: the plan is an argument.
 *
 * A field < 0 keeps the library's own choice; a NULL plan keeps all of them (the
 * *_planned call is then exactly its nvfp4.h counterpart).  A plan that names a
 * layout the library does not build returns NVFP4_ERROR_INVALID_VALUE before any
 * HIP call.  The workspace a call needs depends on the plan: size it with the
 * matching *_planned query.
 */
#ifndef NVFP4_PLAN_H
#define NVFP4_PLAN_H

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    /* Activation rows from which nvfp4_gemm runs the LDS-tiled MFMA GEMM
     * instead of the weight-streaming GEMV (default 65; >= 1). */
    int gemm_min_m;
    /* Largest M (per 32-row chunk) of the 4x4x4-block GEMV (default 4; 0..8). */
    int gemv_small_max;
    /* GEMV weight tiles per wave: 4x4x4-block GEMV {1, 2, 4, 8 (M <= 4)};
     * 16x16 GEMV {1, 2, 4 (M <= 16)}. */
    int gemv_tiles;
    /* GEMV waves per workgroup: 4x4x4-block GEMV 1..8; 16x16 GEMV {4, 8, or 16
     * with 16 < M <= 32 and at most 2 tiles per wave}. */
    int gemv_waves;
    /* LDS budget (KiB, 8..160) of the 4x4x4-block GEMV's staged activations. */
    int gemv_lds_kib;
    /* GEMV K parts across workgroups (>= 1; capped at the K steps). */
    int gemv_splits;
    /* nvfp4_gemm_w4a4_bf16: 1 quantizes the activations inside the product
     * kernel's activation loads (GEMV staging with at most 2 tiles per wave, or
     * the MFMA GEMM's tile loads), 0 in one pass into the workspace first. */
    int w4a4_fuse;
    /* nvfp4_grouped_gemm: average rows per expert from which the MFMA tile
     * kernel replaces the weight-streaming grouped GEMV (default 32; >= 0). */
    int grouped_mfma_min_rows;
    /* GEMV K parts inside one workgroup, summed in LDS (16x16 GEMV, K % 256
     * == 0; gemv_waves = tile groups * parts).  Built layouts (tiles, waves,
     * parts): one activation tile (M <= 16) (2,8,4) (2,8,2) (1,16,4) (1,8,2),
     * and for M <= 8 also (2,16,8) (1,16,8) (2,8,8); two activation tiles
     * (16 < M <= 32) (1,16,2). */
    int gemv_kparts;
    /* Waves per workgroup of the grouped GEMV, which share one staged copy of
     * the chunk's activation rows: 4, 8 or 16. */
    int grouped_gemv_waves;
} nvfp4_plan_t;

/* Every field set to -1 (the library's own choice). */
void nvfp4_plan_default(nvfp4_plan_t *plan);

size_t nvfp4_gemm_workspace_size_planned(const nvfp4_plan_t *plan, int a_dtype, int64_t M,
                                         int64_t N, int64_t K, int64_t n_out);
int nvfp4_gemm_planned(const nvfp4_plan_t *plan, int a_dtype, const void *a,
                       const uint8_t *a_scales, int64_t M, int64_t N, int64_t K,
                       const uint8_t *w_codes, const uint8_t *w_scales, const int32_t *row_idx,
                       int64_t n_out, int out_dtype, void *out, void *workspace,
                       size_t workspace_bytes, void *stream);

size_t nvfp4_gemm_w4a4_bf16_workspace_size_planned(const nvfp4_plan_t *plan, int64_t M,
                                                   int64_t N, int64_t K, int64_t n_out);
int nvfp4_gemm_w4a4_bf16_planned(const nvfp4_plan_t *plan, const uint16_t *a, int64_t M,
                                 int64_t N, int64_t K, const uint8_t *w_codes,
                                 const uint8_t *w_scales, const int32_t *row_idx, int64_t n_out,
                                 int out_dtype, void *out, void *workspace,
                                 size_t workspace_bytes, void *stream);

int nvfp4_grouped_gemm_planned(const nvfp4_plan_t *plan, const uint16_t *a, int64_t a_rows,
                               int64_t K, const int32_t *gather_idx,
                               const int32_t *expert_offsets, int64_t E, int64_t R, int64_t N,
                               const uint8_t *w_codes, const uint8_t *w_scales,
                               const float *row_scale, int epilogue, uint16_t *out,
                               void *workspace, size_t workspace_bytes, void *stream);

int nvfp4_grouped_gemm_scaled_planned(const nvfp4_plan_t *plan, const uint16_t *a,
                                      int64_t a_rows, int64_t K, const int32_t *gather_idx,
                                      const int32_t *expert_offsets, int64_t E, int64_t R,
                                      int64_t N, const uint8_t *w_codes, const uint8_t *w_scales,
                                      const float *w_global_scales, const float *row_scale,
                                      int epilogue, uint16_t *out, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* nvfp4_gemm_tiled with a plan.  4x4x4-block kernel (M <= gemv_small_max,
 * default 4, at most 8): one tile of 16 rows per wave (two with M <= 4), 1..8
 * waves; with gemv_kparts in {2, 4, 8, 16} (M <= 4, one tile per wave)
 * gemv_waves = tile groups x parts, at most 16.  16x16 kernel: gemv_tiles
 * {1, 2, 4 (M <= 16)}, gemv_waves {4, 8, or 16 with 16 < M <= 32}, or the
 * K-parts layouts of gemv_kparts.  gemv_splits and gemv_lds_kib as for
 * nvfp4_gemm. */
size_t nvfp4_gemm_tiled_workspace_size_planned(const nvfp4_plan_t *plan, int a_dtype, int64_t M,
                                               int64_t N, int64_t K);
int nvfp4_gemm_tiled_planned(const nvfp4_plan_t *plan, int a_dtype, const void *a,
                             const uint8_t *a_scales, int64_t M, int64_t N, int64_t K,
                             const uint8_t *w_tiled, int out_dtype, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

int nvfp4_grouped_gemm_tiled_planned(const nvfp4_plan_t *plan, const uint16_t *a,
                                     int64_t a_rows, int64_t K, const int32_t *gather_idx,
                                     const int32_t *expert_offsets, int64_t E, int64_t R,
                                     int64_t N, const uint8_t *w_tiled,
                                     const float *w_global_scales, const float *row_scale,
                                     int epilogue, uint16_t *out, void *workspace,
                                     size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_PLAN_H */
