/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 weight-quantized linear layer.
 *
 * NVFP4 block format ("Serving Qwen3.8-27B in 4-bit with a masked speculative
 * decoding head", section "What the artifact is"): every element is a 4-bit
 * e2m1 float (sign, 2 exponent bits with bias 1, 1 mantissa bit; values
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}) and each run of 16 consecutive K-elements
 * shares one FP8 E4M3 scale (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; "What 350+ Experiments Taught Us About Serving Qwen 3.6 35B-A3B",
 * section 3 "KV cache and memory capacity").  An element's value is
 * e2m1(code) * e4m3(scale); the product is exact in bf16.
 *
 * Layout of an NVFP4 matrix with R rows and K columns ("NF4W(R, K)"):
 *   codes  uint8 [R][K/2], row-major; element 2j of a row sits in the low
 *          nibble of byte j, element 2j+1 in the high nibble;
 *   scales uint8 [R][K/16], row-major E4M3 codes; byte b scales elements
 *          16b .. 16b+15 of its row.  No swizzle, no per-tensor scale.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers (HBM) owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after the call
 *     returns, and keeps no state between calls (calls are re-entrant).
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Every call only enqueues work on `stream` and returns without
 *     synchronising.  A failure to launch returns NVFP4_ERROR_LAUNCH; faults
 *     during execution surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call: null pointers,
 *     sizes (> 0, K % 32 == 0 unless stated), 16-byte alignment of every
 *     array base, and workspace size.  Violations return an error status and
 *     touch no device state.  Properties of device-resident contents (row
 *     indices sorted, offsets non-decreasing, expert ids in range) are
 *     preconditions and are not checked.
 *   - Inputs are never written.  Outputs are fully overwritten and must not
 *     alias an input.
 *   - Results are bit-identical from run to run on the same device, shape
 *     and inputs: reductions use a fixed order and no floating-point atomics.
 *   - bf16 values are passed as their uint16_t bit patterns.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_SUCCESS = 0,
    NVFP4_ERROR_INVALID_VALUE = 1, /* null pointer, non-positive size, misalignment */
    NVFP4_ERROR_NOT_SUPPORTED = 2, /* e.g. K not a multiple of 32, unsupported dtype */
    NVFP4_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    NVFP4_ERROR_LAUNCH = 4         /* a kernel launch failed (hipGetLastError) */
} nvfp4_status_t;

typedef enum {
    NVFP4_BF16 = 0,  /* bfloat16 */
    NVFP4_FP32 = 1,  /* IEEE binary32 */
    NVFP4_NVFP4 = 2  /* NVFP4 codes + E4M3 scales */
} nvfp4_dtype_t;

typedef enum {
    NVFP4_EPI_NONE = 0,   /* out = h */
    NVFP4_EPI_SWIGLU = 1  /* out[:, i] = silu(h[:, i]) * h[:, i + N/2], i < N/2 */
} nvfp4_epilogue_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *nvfp4_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int nvfp4_version(void);

/*
 * Dequantize an NVFP4 matrix NF4W(N, K) to bf16 out[N][K]:
 *   out[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k/16])
 * (format: "Serving Qwen3.8-27B in 4-bit ...", section "What the artifact
 * is").  The result is exact; the sign of zero follows the code's sign bit
 * times the scale's sign.  A NaN scale code (0x7F, 0xFF) gives NaN elements.
 * K % 32 == 0.
 */
int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                     uint16_t *out, void *stream);

/*
 * Quantize bf16 activations x[M][K] to NVFP4 for the W4A4 path ("52.6% more
 * tokens, 1.53x less GPU time: production inference with Minima and Rafay":
 * NVFP4 W4A4 execution).  Per row and per block of 16 elements:
 *   a     = max |x|,
 *   scale = a/6 rounded to the nearest E4M3 value, ties to even code,
 *           saturating to 448 (code 0x7E) -- scales are never negative;
 *   code  = sign of x (negative zero included) | index of the e2m1 magnitude
 *           nearest to |x|/scale, ties to the even index, saturating at 6;
 *           a zero scale gives magnitude 0.
 * Outputs: codes[M][K/2], scales[M][K/16] (the NF4W(M, K) layout).  The
 * result is unique and bit-exact.  Non-finite inputs are outside the
 * contract, but they stay inside their block: a block holding a NaN gets the
 * E4M3 NaN scale code 0x7F (it decodes to NaN) and codes that keep only their
 * sign bits; an infinity saturates like any value above 6*448.  K % 32 == 0.
 */
int nvfp4_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales,
                   void *stream);

/*
 * Bytes of device workspace nvfp4_gemm needs for this activation dtype and
 * shape (0 if none).  n_out is the number of output columns (N, or the
 * row_idx length).  Pure function of its arguments.
 */
size_t nvfp4_gemm_workspace_size(int a_dtype, int64_t M, int64_t N, int64_t K, int64_t n_out);

/*
 * NVFP4 linear layer, y = a . W^T with W = NF4W(N, K) and fp32 accumulation:
 *   out[m][j] = sum_k a[m][k] * w[n_j][k],   n_j = row_idx ? row_idx[j] : j.
 *   a_dtype == NVFP4_BF16  : W4A16 -- a is bf16 [M][K], a_scales must be NULL
 *                            ("What 350+ Experiments ...", section 1).
 *   a_dtype == NVFP4_NVFP4 : W4A4 -- a is codes [M][K/2], a_scales is
 *                            [M][K/16] (output of nvfp4_quantize).
 *   row_idx (optional, int32 [n_out], sorted ascending, unique, < N): compute
 *            only those weight rows; the output is compact [M][n_out] in
 *            row_idx order ("Serving Qwen3.8-27B in 4-bit ...", section "The
 *            masked head trick").  NULL means all rows, n_out must equal N.
 *   out_dtype: NVFP4_BF16 (round to nearest even) or NVFP4_FP32.
 * Decode shapes (small M) stream the weights once with a split-K GEMV;
 * large M uses an MFMA GEMM.  workspace: >= nvfp4_gemm_workspace_size(...)
 * bytes of device memory (may be NULL when that is 0).
 */
int nvfp4_gemm(int a_dtype, const void *a, const uint8_t *a_scales, int64_t M, int64_t N,
               int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
               const int32_t *row_idx, int64_t n_out, int out_dtype, void *out,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * nvfp4_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same operation, arguments, results (bit-identical
 * to nvfp4_gemm) and status codes otherwise.  The workspace nvfp4_gemm would
 * take lives in a device array inside the library, nvfp4_noalloc_scratch_bytes()
 * = 64 MiB on each GPU, held until the process ends: a call whose
 * nvfp4_gemm_workspace_size exceeds it returns NVFP4_ERROR_WORKSPACE before
 * any launch.  The call allocates nothing (no hipMalloc, no library
 * allocator); its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress).  Every call on one GPU shares its array: calls
 * that overlap in time on one GPU (different streams, or host threads) race
 * and must be serialised by the caller.  Nothing in the array needs to start
 * at zero: each call writes every workspace byte it reads.
 */
size_t nvfp4_noalloc_scratch_bytes(void);
int nvfp4_gemm_noalloc(int a_dtype, const void *a, const uint8_t *a_scales, int64_t M, int64_t N,
                       int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
                       const int32_t *row_idx, int64_t n_out, int out_dtype, void *out,
                       void *stream);

/*
 * Tiled NVFP4 weights ("NF4T"): the same matrix NF4W(N, K), bytes reordered
 * once when the weights are loaded so that the weight-streaming kernels read
 * every step of a wave as contiguous, fully used runs, the scales in the same
 * stream as the codes (the pages' Marlin-class kernels also take weights
 * repacked offline: "Serving Qwen3.8-27B in 4-bit ...", sections "What the
 * artifact is" and "The masked head trick").  Rows are grouped in tiles of 16
 * and K in steps of 256 elements; block (t, s) is 2,304 bytes at offset
 * (t * S + s) * 2304, S = ceil(K / 256):
 *   bytes [1024 h + 16 L, +16), h = 0, 1, L = 16 q + n (n, q < 16, 4): the
 *     code bytes of row 16 t + n, elements 256 s + 64 q + 32 h .. + 31, in
 *     the row-major nibble order;
 *   bytes [2048 + 4 L, +4): that row's scale bytes of elements
 *     256 s + 64 q .. + 63 (four blocks of 16).
 * Rows past N and elements past K hold zero codes and zero scales.  The array
 * holds nvfp4_tiled_weight_bytes(N, K) = ceil(N/16) * S * 2304 bytes, equal to
 * the row-major bytes when N % 16 == 0 and K % 256 == 0.
 */
size_t nvfp4_tiled_weight_bytes(int64_t N, int64_t K);

/*
 * Write the tiled layout of NF4W(N, K) (codes [N][K/2], scales [N][K/16]) to
 * w_tiled, every byte written: a pure byte permutation plus zero padding.
 * row_idx (optional, int32 [n_rows], each < N): tile only those rows, in that
 * order -- tiled row r is row row_idx[r] -- as for a masked head whose id set
 * is fixed when the weights are loaded ("Serving Qwen3.8-27B in 4-bit ...",
 * section "The masked head trick": the top 32,768 of 248,320 ids).  NULL
 * means all rows (n_rows must equal N).  w_tiled holds
 * nvfp4_tiled_weight_bytes(n_rows, K) bytes.  K % 32 == 0.
 */
int nvfp4_tile_weight(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                      const int32_t *row_idx, int64_t n_rows, uint8_t *w_tiled, void *stream);

/*
 * nvfp4_gemm on tiled weights of N rows (all rows of the tiled matrix; a row
 * subset is tiled as its own matrix): out[m][n] = sum_k a[m][k] * w[n][k],
 * out [M][N] in out_dtype, a_dtype / a / a_scales as in nvfp4_gemm.  Decode
 * shapes stream the weights with the split-K GEMV, 32 activation rows per
 * launch; large M runs the MFMA GEMM, as nvfp4_gemm does.
 * Same products, fp32 accumulation, tolerance and run-to-run determinism as
 * nvfp4_gemm.  workspace: >= nvfp4_gemm_tiled_workspace_size(a_dtype, M, N,
 * K) bytes (may be NULL when that is 0).  K % 32 == 0.
 */
size_t nvfp4_gemm_tiled_workspace_size(int a_dtype, int64_t M, int64_t N, int64_t K);
int nvfp4_gemm_tiled(int a_dtype, const void *a, const uint8_t *a_scales, int64_t M, int64_t N,
                     int64_t K, const uint8_t *w_tiled, int out_dtype, void *out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * W4A4 linear layer from bf16 activations: the activation quantizer fused into
 * the product ("52.6% more tokens, 1.53x less GPU time ...": NVFP4 W4A4
 * execution).  Bit-identical to nvfp4_quantize(a) followed by nvfp4_gemm
 * with a_dtype = NVFP4 (same arguments otherwise: row_idx, n_out, out_dtype).
 * Very small M quantizes every 16-element block while the GEMV stages the
 * activations, so the codes never go to memory; otherwise one pass writes the
 * activations quantized and dequantized (bf16, exact) into the workspace and
 * the bf16-activation GEMV or MFMA GEMM runs on them.
 * workspace: >= nvfp4_gemm_w4a4_bf16_workspace_size(M, N, K, n_out) bytes.
 * K % 32 == 0.
 */
size_t nvfp4_gemm_w4a4_bf16_workspace_size(int64_t M, int64_t N, int64_t K, int64_t n_out);
int nvfp4_gemm_w4a4_bf16(const uint16_t *a, int64_t M, int64_t N, int64_t K,
                         const uint8_t *w_codes, const uint8_t *w_scales,
                         const int32_t *row_idx, int64_t n_out, int out_dtype, void *out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Two-level NVFP4.  The deployed NVFP4 checkpoints come from NVFP4
 * quantization tools ("What 350+ Experiments ...", section 1 and its
 * sources); a tensor then carries, above its per-16 E4M3 scales, one positive
 * fp32 global scale g, and an element is e2m1(code) * e4m3(scale) * g.  g is
 * a DEVICE pointer to one float (4-byte aligned).
 *
 * nvfp4_quantize_scaled: activations with a given g (e.g. a calibrated static
 * scale): y = fl32(x / g) (binary32 division, nearest even), then exactly the
 * nvfp4_quantize rule on y.  g = 1 reproduces nvfp4_quantize.  Bit-exact.
 *
 * nvfp4_quantize_weight: offline weight quantizer, bf16 w [N][K] -> codes,
 * scales and *global_scale = fl32(amax / 2688) (2688 = 6 * 448, so the
 * block holding max |w| gets scale 448; 1 for an all-zero tensor), then
 * nvfp4_quantize_scaled with that g.  Bit-exact.  workspace: >=
 * nvfp4_quantize_weight_workspace_size(N, K) bytes.
 *
 * nvfp4_dequantize_scaled: out[n][k] = bf16(fl32(e2m1 * e4m3 * g)) (the first
 * product is exact; one binary32 rounding, then bf16, nearest even).
 *
 * nvfp4_gemm_scaled: nvfp4_gemm of two-level operands,
 *   out = (a . W^T) * (a_g * w_g),
 * the factor fl32(a_g * w_g) applied once to the fp32 sums (NULL pointer: 1;
 * a_global_scale only with NVFP4 activations).  Same shapes, workspace
 * (nvfp4_gemm_workspace_size) and tolerance as nvfp4_gemm.  K % 32 == 0 for all.
 */
int nvfp4_quantize_scaled(const uint16_t *x, int64_t M, int64_t K, const float *global_scale,
                          uint8_t *codes, uint8_t *scales, void *stream);
size_t nvfp4_quantize_weight_workspace_size(int64_t N, int64_t K);
int nvfp4_quantize_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                          uint8_t *scales, float *global_scale, void *workspace,
                          size_t workspace_bytes, void *stream);
int nvfp4_dequantize_scaled(const uint8_t *codes, const uint8_t *scales,
                            const float *global_scale, int64_t N, int64_t K, uint16_t *out,
                            void *stream);
int nvfp4_gemm_scaled(int a_dtype, const void *a, const uint8_t *a_scales,
                      const float *a_global_scale, int64_t M, int64_t N, int64_t K,
                      const uint8_t *w_codes, const uint8_t *w_scales,
                      const float *w_global_scale, const int32_t *row_idx, int64_t n_out,
                      int out_dtype, void *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * Draft proposal from a head's logits ("Serving Qwen3.8-27B in 4-bit ...",
 * section "The masked head trick": the draft proposes tokens only from the
 * kept rows of the head).  For each row m of logits (fp32 [M][n]) the k best
 * entries, best first:
 *   values[m][i] = logits[m][c_i],  ids[m][i] = ids_map ? ids_map[c_i] : c_i,
 * ordered by larger value, then smaller column c (the rank in the mask);
 * -0 ranks below +0.  The result is unique and bit-exact.  NaN logits are
 * outside the contract (they are ranked by their bit patterns).
 * 1 <= k <= min(n, 256), n <= INT32_MAX, M <= 65535.  ids_map (optional,
 * int32 [n]) maps columns to token ids.  values fp32 [M][k], ids int32 [M][k].
 * workspace: >= nvfp4_topk_workspace_size(M, n, k) bytes (0 for n <= 2048).
 */
size_t nvfp4_topk_workspace_size(int64_t M, int64_t n, int64_t k);
int nvfp4_topk(const float *logits, int64_t M, int64_t n, int64_t k, const int32_t *ids_map,
               float *values, int32_t *ids, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Masked draft head with its proposal ("Serving Qwen3.8-27B in 4-bit ...",
 * section "The masked head trick"): the W4A16 head over the kept rows, then
 * the top-k of each row,
 *   logits[m][j] = sum_k a[m][k] * w[row_idx[j]][k]   (fp32, as nvfp4_gemm),
 *   values/ids   = nvfp4_topk(logits, k, ids_map = row_idx)
 * so ids are weight-row (token) ids.  a is bf16 [M][K]; row_idx as in
 * nvfp4_gemm (NULL: every row, n_out = N).  The logits stay in the workspace
 * and are not returned.  1 <= k <= min(n_out, 256), M <= 65535, K % 32 == 0.
 * workspace: >= nvfp4_head_topk_workspace_size(M, N, K, n_out, k) bytes.
 */
size_t nvfp4_head_topk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t n_out,
                                      int64_t k);
int nvfp4_head_topk(const uint16_t *a, int64_t M, int64_t N, int64_t K, const uint8_t *w_codes,
                    const uint8_t *w_scales, const int32_t *row_idx, int64_t n_out, int64_t k,
                    float *values, int32_t *ids, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * FP8 E4M3 KV cache ("What 350+ Experiments ...", section 3 "KV cache and
 * memory capacity": the key/value cache held as FP8 E4M3 in 16-token pages).
 * A cache is uint8 [num_slots][W] (W = heads * head size of the keys or of
 * the values); slot = page * page_size + position in the page, so the paged
 * layout [pages][page_size][W] is the same array.  One fp32 scale per cache
 * (finite, >= 2^-126).
 *
 * nvfp4_kv_store_e4m3: token rows x (bf16 [T][W]) into their slots,
 *   cache[slot_mapping[t]][w] = E4M3(fl32(x[t][w] / scale)),
 * fl32 = binary32 division, nearest even; E4M3 = nearest code, ties to the
 * even code, saturating to +-448, sign kept.  The result is bit-exact.  The
 * cache is updated in place (the one exception to "outputs are fully
 * overwritten"): slot_mapping[t] < 0 (padding) or >= num_slots leaves it
 * untouched; slots must be distinct.  A NaN element is stored as the NaN code
 * of its sign (0x7F / 0xFF); infinities saturate to +-448.  W % 16 == 0.
 *
 * nvfp4_kv_load_e4m3: B sequences back to bf16 out [B][max_len][W],
 *   out[b][i][w] = bf16(fl32(e4m3(cache[s][w]) * scale)),
 *   s = block_table[b][i / page_size] * page_size + i % page_size,
 * for i < seq_lens[b] (block_table int32 [B][max_pages], seq_lens int32 [B]);
 * rows i >= seq_lens[b], and rows whose slot falls outside the cache, are
 * zero.  Bit-exact.  W % 16 == 0.
 */
int nvfp4_kv_store_e4m3(const uint16_t *x, int64_t T, int64_t W, const int32_t *slot_mapping,
                        float scale, uint8_t *cache, int64_t num_slots, void *stream);
int nvfp4_kv_load_e4m3(const uint8_t *cache, int64_t num_slots, int64_t W,
                       const int32_t *block_table, const int32_t *seq_lens, int64_t B,
                       int64_t max_pages, int64_t page_size, int64_t max_len, float scale,
                       uint16_t *out, void *stream);

/*
 * Routing preparation for a routed mixture-of-experts layer ("What 350+
 * Experiments ...", section 1: a routed-expert model).  topk_ids int32
 * [T][topk] holds, for each token, the experts it is routed to (each in
 * [0, E)).  A stable counting sort by expert produces:
 *   expert_offsets int32 [E+1]: rows of expert e are offsets[e] .. offsets[e+1]-1,
 *                               offsets[E] = T*topk;
 *   gather_idx     int32 [T*topk]: token whose activation row r reads;
 *   slot_pos       int32 [T*topk]: row that assignment p = t*topk + j landed in;
 *   row_gates      optional fp32 [T*topk]: row_gates[slot_pos[p]] = gates[p], the
 *                  per-token gate weights (gates, fp32 [T][topk]) in row order,
 *                  ready to scale the rows of the down projection.  Both NULL
 *                  or both given.
 * Rows of one expert keep ascending p.  The result is unique.  topk <= 32,
 * E <= 1024.  Ids outside [0, E) are a precondition violation: such
 * assignments are skipped (never written out of bounds) and the outputs are
 * then unspecified.  workspace: >= nvfp4_moe_align_workspace_size(T, topk, E)
 * bytes of device memory.
 */
size_t nvfp4_moe_align_workspace_size(int64_t T, int64_t topk, int64_t E);
int nvfp4_moe_align(const int32_t *topk_ids, const float *gates, int64_t T, int64_t topk,
                    int64_t E, int32_t *expert_offsets, int32_t *gather_idx,
                    int32_t *slot_pos, float *row_gates, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Bytes of device workspace nvfp4_grouped_gemm needs (0 if none). */
size_t nvfp4_grouped_gemm_workspace_size(int64_t R, int64_t E, int64_t N, int64_t K);

/*
 * Grouped W4A16 GEMM over experts ("What 350+ Experiments ...", sections 1
 * and 7: NVFP4 expert weights run by a grouped mixture-of-experts kernel).
 * Row r < R belongs to the expert e with offsets[e] <= r < offsets[e+1]
 * (expert_offsets is device int32 [E+1], offsets[0] = 0, offsets[E] = R,
 * non-decreasing).  It reads activation row src = gather_idx ? gather_idx[r]
 * : r of a (bf16 [a_rows][K]) and computes, with fp32 accumulation,
 *   h[n] = sum_k a[src][k] * w_e[n][k],   n < N,
 * where w_e is NF4W(N, K) of expert e (w_codes [E][N][K/2], w_scales
 * [E][N][K/16]).  Epilogue: NVFP4_EPI_NONE writes h (width N);
 * NVFP4_EPI_SWIGLU writes silu(h[i]) * h[i + N/2] (width N/2; the first half
 * of each expert's rows is the gate projection, the second half the up
 * projection; N even).  If row_scale (fp32 [R]) is given, the row is then
 * multiplied by row_scale[r].  The result is rounded to bf16 into out
 * [R][width].  K % 32 == 0.
 */
int nvfp4_grouped_gemm(const uint16_t *a, int64_t a_rows, int64_t K, const int32_t *gather_idx,
                       const int32_t *expert_offsets, int64_t E, int64_t R, int64_t N,
                       const uint8_t *w_codes, const uint8_t *w_scales, const float *row_scale,
                       int epilogue, uint16_t *out, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * nvfp4_grouped_gemm of two-level expert weights.  The MoE checkpoints the
 * pages deploy come from NVFP4 quantization tools ("What 350+ Experiments
 * ...", section 1); each expert tensor then carries one positive fp32 global
 * scale above its per-16 E4M3 scales (see the two-level functions above;
 * nvfp4_quantize_weight run per expert writes them).  w_global_scales is a
 * DEVICE fp32 array [E] (4-byte aligned; NULL means 1 for every expert).  The
 * fp32 sums of expert e are multiplied by w_global_scales[e] before the
 * epilogue:
 *   h[n] = fl32( w_global_scales[e] * sum_k a[src][k] * w_e[n][k] ),
 * then SwiGLU (the gate and up halves of a fused W1 share their expert's
 * scale), row_scale and the bf16 rounding exactly as nvfp4_grouped_gemm.
 * All scales 1 (or NULL) gives nvfp4_grouped_gemm's output bit for bit.
 * Other arguments, errors and workspace as nvfp4_grouped_gemm.
 */
int nvfp4_grouped_gemm_scaled(const uint16_t *a, int64_t a_rows, int64_t K,
                              const int32_t *gather_idx, const int32_t *expert_offsets, int64_t E,
                              int64_t R, int64_t N, const uint8_t *w_codes,
                              const uint8_t *w_scales, const float *w_global_scales,
                              const float *row_scale, int epilogue, uint16_t *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * nvfp4_grouped_gemm_scaled on tiled expert weights: w_tiled is
 * nvfp4_tile_weight of the stacked E*N-row matrix (codes [E*N][K/2], scales
 * [E*N][K/16]; N % 16 == 0, so expert e's N/16 tiles follow expert e-1's),
 * nvfp4_tiled_weight_bytes(E*N, K) bytes ("What 350+ Experiments ...",
 * section 7: NVFP4 expert weights served by a grouped kernel).
 * w_global_scales may be NULL (single-level experts).  Same operation,
 * arguments, results (bit-identical to the row-major call of the same kernel
 * choice), errors and workspace as nvfp4_grouped_gemm_scaled.
 */
int nvfp4_grouped_gemm_tiled(const uint16_t *a, int64_t a_rows, int64_t K,
                             const int32_t *gather_idx, const int32_t *expert_offsets, int64_t E,
                             int64_t R, int64_t N, const uint8_t *w_tiled,
                             const float *w_global_scales, const float *row_scale, int epilogue,
                             uint16_t *out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Combine the per-slot expert outputs of a routed layer ("What 350+
 * Experiments ...", section 1: each token's output is the gate-weighted sum
 * over the experts it was routed to; the gate weights are applied by the
 * down projection's row_scale, so this step only adds):
 *   out[t][c] = bf16( sum_{j < topk} y[slot_pos[t*topk + j]][c] )
 * summed in fp32 in slot order.  y is bf16 [R][H] with R = T*topk, out is
 * bf16 [T][H].  H % 8 == 0.
 */
int nvfp4_moe_combine(const uint16_t *y, const int32_t *slot_pos, int64_t T, int64_t topk,
                      int64_t H, uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
