// launch.h -- host-side launchers of the NVFP4 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Compute units of an MI355X; launch plans are a pure function of the shape
// and this constant, so workspace queries need no device.
constexpr int kNumCUs = 256;

int launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                      uint16_t* out, hipStream_t stream);
int launch_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                    hipStream_t stream);
// out = dequantize(quantize(x)) in bf16 (exact), without the codes in memory.
int launch_fakequant(const uint16_t* x, int64_t M, int64_t K, uint16_t* out, hipStream_t stream);

// Tiled NVFP4 weights (tile.hip): blocks of 16 rows x 256 elements, 2,304
// bytes each (two 1 KB halves of codes in lane order, then 256 B of scales),
// tile-major; rows past N and elements past K are zero.
constexpr int kTileRows = 16;
constexpr int kTileStep = 256;
constexpr int kTileBlockBytes = 2304;
size_t tiled_weight_bytes(int64_t N, int64_t K);
// Tiled rows r < R are row-major rows row_idx[r] (r when row_idx is null).
int launch_tile_weight(const uint8_t* codes, const uint8_t* scales, const int32_t* row_idx,
                       int64_t R, int64_t K, uint8_t* out, hipStream_t stream);

// Two-level NVFP4 (per-tensor fp32 scale g, a device scalar).  Quantize with
// a given g; the offline weight quantizer (g from the tensor's amax, written
// to *g; kAbsmaxParts partial maxima in workspace); dequantize with g.
constexpr int kAbsmaxParts = 256;
int launch_quantize_scaled(const uint16_t* x, int64_t M, int64_t K, const float* g,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);
size_t quantize_weight_workspace_bytes();
int launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* scales, float* g, void* workspace, hipStream_t stream);
int launch_dequantize_scaled(const uint8_t* codes, const uint8_t* scales, const float* g,
                             int64_t N, int64_t K, uint16_t* out, hipStream_t stream);

// Output multiplier of a product of two-level tensors: alpha = *a * *w, each
// factor 1 when its pointer is null (then no multiply happens at all).
struct Alpha {
  const float* a = nullptr;
  const float* w = nullptr;
};

// Launch-plan overrides of the tuning entry points (include/nvfp4_plan.h):
// every field < 0 keeps the plan's own choice.  The product entry points pass
// the all-default value, so their plans stay a pure function of the shape.
struct PlanOverride {
  int gemm_min_m = -1;             // rows of M from which the MFMA GEMM runs
  int gemv_small_max = -1;         // largest M of the 4x4x4-block GEMV (0..8)
  int gemv_tiles = -1;             // weight tiles per wave
  int gemv_waves = -1;             // waves per workgroup
  int gemv_lds_kib = -1;           // LDS budget of the 4x4x4 kernel's staged activations
  int gemv_splits = -1;            // K parts across workgroups
  int gemv_kparts = -1;            // K parts inside a workgroup (16x16 GEMV, K % 256 == 0)
  int w4a4_fuse = -1;              // W4A4 from bf16: quantize inside the kernel (1) or in a pass (0)
  int grouped_mfma_min_rows = -1;  // average rows per expert from which the grouped MFMA runs
  int grouped_gemv_waves = -1;     // waves per workgroup of the grouped GEMV (4, 8, 16)
};

struct GemvPlan {
  bool small;  // M <= 4: 4x4x4-block kernel (tiles of 4 rows)
  int mt;  // 16-row activation tiles (M <= 16 * mt)
  int tr;  // 16-row weight tiles per wave
  int nw;  // waves per workgroup (each streams its own weight tiles)
  int z;   // split-K across workgroups (fp32 partials + reduce kernel)
  int kp;  // K parts inside a workgroup (nw = tile groups * kp), summed in LDS
};

// tiled: the plan of launch_gemv_tiled (16x16 kernel only, K parts across
// workgroups only).
GemvPlan plan_gemv(int64_t M, int64_t n_out, int64_t K, int num_cus,
                   const PlanOverride& ov = PlanOverride{}, bool tiled = false);
// Whether the override's GEMV fields name a layout that exists for this M.
bool gemv_override_valid(int64_t M, int64_t K, const PlanOverride& ov);
size_t gemv_workspace_bytes(const GemvPlan& p, int64_t M, int64_t n_out);
// fakequant: x is bf16 and every 16-element block is quantized to NVFP4 and
// dequantized while it is staged (the W4A4 product with the activation
// quantizer fused in; one or two weight tiles per wave).
int launch_gemv(const GemvPlan& p, const uint16_t* x, int64_t M, int64_t K, const uint8_t* wc,
                const uint8_t* ws, const int32_t* row_idx, int64_t n_out, bool out_f32,
                void* out, void* workspace, hipStream_t stream, Alpha alpha = {},
                bool fakequant = false);
// The same product with tiled weights (wt: tiled_weight_bytes(N, K), all N
// rows; no row_idx and no fused quantizer).
int launch_gemv_tiled(const GemvPlan& p, const uint16_t* x, int64_t M, int64_t K,
                      const uint8_t* wt, int64_t N, bool out_f32, void* out, void* workspace,
                      hipStream_t stream, Alpha alpha = {});

// Large-M path: LDS-tiled MFMA GEMM, 256 x 256 output tiles.  a is bf16 [M][K];
// with GemmA::kFakeQuant its tiles are quantized to NVFP4 and dequantized as
// they are loaded (the W4A4 product from bf16 activations).  The tiles of a
// last, partly filled round (or all tiles, when they cannot fill the chip
// once) share one round of workgroups: their (tile, K step) work is cut into
// `parts` equal contiguous ranges, one per workgroup, each range's pieces of
// a tile (segments) writing fp32 tile-local partials to workspace
// (gemm_workspace_bytes of it), summed in K order by a second kernel.
struct GemmSplitPlan {
  int64_t full;  // tiles run whole
  int64_t tail;  // tiles shared by `parts` workgroups (0: none)
  int parts;
  int max_seg;   // most segments of one tail tile (partial slots per tile)
  bool own_launch;  // the shared round is a launch of its own (every tile is shared);
                    // otherwise its workgroups follow the whole tiles' in one launch,
                    // one segment each
};
GemmSplitPlan gemm_split_plan(int64_t M, int64_t n_out, int64_t K, int num_cus);
size_t gemm_workspace_bytes(int64_t M, int64_t n_out, int64_t K, int num_cus);
enum class GemmA { kBf16, kFakeQuant };
// tiled: wc is the tiled weights (tile.hip), ws and row_idx unused.
int launch_gemm(GemmA mode, const void* a, int64_t M, int64_t K, const uint8_t* wc,
                const uint8_t* ws, const int32_t* row_idx, int64_t n_out, bool out_f32, void* out,
                void* workspace, hipStream_t stream, Alpha alpha = {}, bool tiled = false);

// Top-k of each row of fp32 logits [M][n] (k <= kTopkMaxK), best first: larger
// value, then smaller column; -0 below +0.  ids are ids_map[column] (or the
// column).  Rows longer than 2048 need topk_workspace_bytes of workspace.
constexpr int kTopkMaxK = 256;
size_t topk_workspace_bytes(int64_t M, int64_t n, int64_t k);
int launch_topk(const float* logits, int64_t M, int64_t n, int64_t k, const int32_t* ids_map,
                float* values, int32_t* ids, void* workspace, hipStream_t stream);

// FP8 E4M3 KV-cache codec: rows of W elements (W % 16 == 0) between bf16
// tokens and a cache of num_slots code rows.
int launch_kv_store(const uint16_t* x, int64_t T, int64_t W, const int32_t* slot_mapping,
                    float scale, uint8_t* cache, int64_t num_slots, hipStream_t stream);
int launch_kv_load(const uint8_t* cache, int64_t num_slots, int64_t W, const int32_t* block_table,
                   const int32_t* seq_lens, int64_t B, int64_t max_pages, int64_t page_size,
                   int64_t max_len, float scale, uint16_t* out, hipStream_t stream);

}  // namespace nvfp4
