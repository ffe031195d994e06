// moe.h -- launchers of the routed mixture-of-experts kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"

namespace nvfp4 {

constexpr int kMoeMaxExperts = 1024;
// LDS a workgroup may hold on gfx950 (160 KiB per CU).
constexpr size_t kGroupedGemvMaxLds = 160 * 1024;

// Kernel of a grouped GEMM: the weight-streaming GEMV (few rows per expert),
// the MFMA tile (many rows, or a K too long for the GEMV's LDS staging), or
// none (a shape neither kernel takes).
enum class GroupedPath { kGemv, kMfma, kNone };
GroupedPath grouped_path(int64_t a_rows, int64_t K, int64_t E, int64_t R,
                         const PlanOverride& ov = PlanOverride{});

size_t moe_align_workspace_bytes(int64_t T, int64_t topk, int64_t E);
int launch_moe_align(const int32_t* ids, const float* gates, int64_t T, int64_t topk, int64_t E,
                     int32_t* offsets, int32_t* gather_idx, int32_t* slot_pos, float* row_gates,
                     void* workspace, hipStream_t stream);

size_t moe_grouped_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K);
int launch_grouped_gemm(const uint16_t* a, int64_t a_rows, int64_t K, const int32_t* gather,
                        const int32_t* offsets, int64_t E, int64_t R, int64_t N,
                        const uint8_t* wc, const uint8_t* ws, const float* wg,
                        const float* row_scale, bool swiglu, uint16_t* out, void* workspace,
                        hipStream_t stream, const PlanOverride& ov = PlanOverride{},
                        bool tiled = false);  // wc: tiled experts (tile.hip), ws unused

int launch_moe_combine(const uint16_t* y, const int32_t* slot_pos, int64_t T, int64_t topk,
                       int64_t H, uint16_t* out, hipStream_t stream);

}  // namespace nvfp4
