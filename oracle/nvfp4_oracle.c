/*
 * nvfp4_oracle.c -- plain, slow, CPU reference for the NVFP4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls, links or includes
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or constant with
 * the HIP implementation.
 *
 * Everything is written as the plain definition of what is computed:
 *   - formats are decoded from their bit fields,
 *   - every rounding decision (scale, code, bf16 output) is taken by exact
 *     comparisons on doubles whose values are exact,
 *   - contractions are plain fp64 sums over k in index order.
 *
 * Sources (web pages; each function names the passage it follows):
 *   [P3] "Serving Qwen3.8-27B in 4-bit with a masked speculative decoding
 *        head", section "What the artifact is": NVFP4 = 4-bit e2m1 elements
 *        with one FP8 scale per 16 consecutive elements;
 *        section "The masked head trick": the draft head reads only a
 *        ranked subset (32,768 of 248,320) of the output rows.
 *   [P4] "What 350+ Experiments Taught Us About Serving Qwen 3.6 35B-A3B",
 *        section 1 "Checkpoint packages and quantisation": W4A16 = 4-bit
 *        weights with 16-bit activations; the model is a routed
 *        mixture-of-experts; section 3 "KV cache and memory capacity": FP8
 *        E4M3 has four exponent bits and three mantissa bits.
 *   [P1] "52.6% more tokens, 1.53x less GPU time: production inference with
 *        Minima and Rafay", opening sections: NVFP4 W4A4 execution
 *        (activations are also cut to NVFP4).
 * Where the pages leave a step open (scale rule amax/6, round-to-nearest-even,
 * satfinite, nibble order, layouts, gate/up order) the reading taken is stated
 * beside the code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Formats                                                                    */
/* ------------------------------------------------------------------------ */

/* e2m1 [P3 "What the artifact is"]: a 4-bit float with 1 sign bit, 2 exponent
 * bits (bias 1) and 1 mantissa bit; exponent field 0 is subnormal (m * 0.5);
 * there is no Inf or NaN.  Code 8 is -0.0. */
double oracle_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3 [P4 section 3]: 1 sign bit, 4 exponent bits, 3 mantissa bits.
 * Reading: the OCP "E4M3FN" variant -- bias 7, exponent field 0 subnormal
 * (m * 2^-9), no infinities, the all-ones exponent with all-ones mantissa
 * (0x7F / 0xFF) is NaN, largest finite value 448. */
double oracle_e4m3_value(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* bf16 bits -> value (exact: bf16 is the top half of an IEEE binary32). */
double oracle_bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* value -> bf16 bits, round to nearest, ties to even, computed directly from
 * the double (no intermediate binary32 rounding).  bf16 keeps 8 significant
 * bits; below 2^-126 the spacing is fixed at 2^-133 (subnormals). */
uint16_t oracle_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v), r, q;
    int e, qexp;
    float f;
    uint32_t u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    qexp = e - 8;                 /* spacing of 8-significant-bit numbers there */
    if (qexp < -133)
        qexp = -133;
    q = ldexp(a, -qexp);          /* exact scaling by a power of two */
    r = nearbyint(q);             /* default mode: nearest, ties to even */
    r = ldexp(r, qexp);
    if (r >= ldexp(1.0, 128))     /* rounds past the largest finite bf16 */
        return (uint16_t)(sign | 0x7F80u);
    f = (float)r;                 /* exact: r is a bf16 value */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* Array form of oracle_bf16_round. */
void oracle_bf16_round_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Dequantization                                                             */
/* ------------------------------------------------------------------------ */

/* Packed-nibble layout (reading; the pages do not fix it): row-major codes
 * [N][K/2], element 2j of a row in the low nibble of byte j and element 2j+1
 * in the high nibble; row-major scales [N][K/16], scale byte b covering
 * elements 16b .. 16b+15. */
static unsigned code_at(const uint8_t *row_codes, int64_t k)
{
    uint8_t byte = row_codes[k >> 1];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

/* w = e2m1(code) * e4m3(scale) [P3 "What the artifact is"].  The product has at
 * most 6 significant bits and magnitude within [2^-10, 2688] (or is zero), so
 * it is exact in bf16; the bf16 bits are returned. */
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                       uint16_t *out)
{
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *rc = codes + n * (K / 2);
        const uint8_t *rs = scales + n * (K / 16);
        for (int64_t k = 0; k < K; ++k) {
            double w = oracle_e2m1_value(code_at(rc, k)) * oracle_e4m3_value(rs[k / 16]);
            out[n * K + k] = oracle_bf16_round(w);
        }
    }
}

/* Tiled NVFP4 weights: the library's own byte order for streaming (not from
 * the pages; its definition is the one stated in the library's public header
 * for nvfp4_tile_weight).  Rows are grouped in tiles of 16, K in steps of 256
 * elements; block (t, s) occupies bytes [(t*S + s)*2304, +2304), S =
 * ceil(K/256).  Written here element by element: code element (r, k) of the
 * row-major matrix goes to
 *     block (r/16, k/256), byte 1024*h + 16*(16*q + r%16) + (k%32)/2,
 *     nibble k%2 (low nibble = even k),
 * with q = (k%256)/64, h = (k%64)/32; scale byte (r, b) of elements
 * 16b .. 16b+15 goes to
 *     block (r/16, b/16), byte 2048 + 4*(16*q + r%16) + b%4, q = (b%16)/4.
 * Every other byte (rows past N, elements past K) is zero.  `out` holds
 * ceil(N/16) * S * 2304 bytes. */
void oracle_tile_weight(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                        uint8_t *out)
{
    int64_t T = (N + 15) / 16, S = (K + 255) / 256;
    memset(out, 0, (size_t)(T * S * 2304));
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t kk = k % 256, q = kk / 64, h = (kk % 64) / 32;
            int64_t off = ((r / 16) * S + k / 256) * 2304 + 1024 * h + 16 * (16 * q + r % 16) +
                          (k % 32) / 2;
            unsigned code = code_at(codes + r * (K / 2), k);
            out[off] |= (uint8_t)(code << (4 * (k % 2)));
        }
        for (int64_t b = 0; b < K / 16; ++b) {
            int64_t q = (b % 16) / 4;
            int64_t off = ((r / 16) * S + b / 16) * 2304 + 2048 + 4 * (16 * q + r % 16) + b % 4;
            out[off] = scales[r * (K / 16) + b];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Quantization                                                               */
/* ------------------------------------------------------------------------ */

/* Scale code for a block whose largest magnitude is a [P3: one FP8 scale per
 * 16 elements; P4 section 3: E4M3].  Reading of the rule: the scale is a/6
 * (6 is the largest e2m1 magnitude) rounded to the nearest E4M3 value, ties to
 * the even code, and saturated to 448 (code 0x7E) when a/6 exceeds it.  Only
 * the 127 finite non-negative codes 0x00..0x7E are candidates.
 *
 * a/6 is never formed: with v(c) the candidate values, "v(c) <= a/6" is tested
 * as 6*v(c) <= a and "a/6 against the midpoint of v(c), v(c+1)" as a against
 * 3*(v(c)+v(c+1)).  Both right-hand sides carry at most 8 significant bits, so
 * every comparison is exact in double.  Non-finite inputs are outside the
 * quantizer's contract; the reading that keeps the damage inside the block is
 * that a NaN maximum takes the E4M3 NaN code 0x7F (the block then decodes to
 * NaN) and an infinite one saturates to 0x7E like any value above 448*6. */
unsigned oracle_scale_code(double a)
{
    unsigned c = 0, next;
    double mid6;
    if (isnan(a))
        return 0x7F;                       /* a block holding a NaN: the NaN code */
    for (unsigned cand = 1; cand <= 0x7E; ++cand)
        if (6.0 * oracle_e4m3_value(cand) <= a)
            c = cand;
    if (c == 0x7E)
        return 0x7E;                       /* at or above 448: satfinite */
    next = c + 1;
    mid6 = 3.0 * (oracle_e4m3_value(c) + oracle_e4m3_value(next));
    if (a < mid6)
        return c;
    if (a > mid6)
        return next;
    return (c & 1u) ? next : c;            /* tie: even code */
}

/* Magnitude index (0..7) of the e2m1 value nearest to |x| / s, for s > 0.
 * Ties go to the even index (mantissa bit 0), values above 6 saturate to
 * index 7.  Comparisons are made as |x| against s * value, exact in double. */
unsigned oracle_e2m1_index(double ax, double s)
{
    unsigned i = 0;
    double mid;
    for (unsigned cand = 1; cand < 8; ++cand)
        if (s * oracle_e2m1_value(cand) <= ax)
            i = cand;
    if (i == 7)
        return 7;
    mid = s * 0.5 * (oracle_e2m1_value(i) + oracle_e2m1_value(i + 1));
    if (ax < mid)
        return i;
    if (ax > mid)
        return i + 1;
    return (i & 1u) ? i + 1 : i;
}

/* One element's 4-bit code for a given scale code: sign bit = sign of x
 * (negative zero included), magnitude index as above; a zero scale gives
 * magnitude 0. */
unsigned oracle_e2m1_encode(uint16_t x_bf16, unsigned scale_code)
{
    double x = oracle_bf16_value(x_bf16);
    double s = oracle_e4m3_value(scale_code);
    unsigned mag = (s == 0.0) ? 0u : oracle_e2m1_index(fabs(x), s);
    return ((signbit(x) ? 1u : 0u) << 3) | mag;
}

/* Array forms of the two rounding steps, for exhaustive checks. */
void oracle_scale_code_array(const double *a, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)oracle_scale_code(a[i]);
}

void oracle_e2m1_encode_array(const uint16_t *x, int64_t n, unsigned scale_code, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)oracle_e2m1_encode(x[i], scale_code);
}

/* NVFP4 quantizer for activations (the W4A4 path of [P1]): per row and per
 * block of 16 consecutive elements, (1) a = max |x|, (2) scale code from a,
 * (3) each element's code against the decoded scale, (4) two codes per byte,
 * element 2j in the low nibble.  x is bf16 [M][K]; codes [M][K/2]; scales
 * [M][K/16].  Non-finite inputs are outside the contract, but a block holding
 * a NaN is confined to itself: its scale code is 0x7F (oracle_scale_code) and
 * every code keeps only its sign bit (no magnitude compares true against a
 * NaN scale). */
void oracle_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < K / 16; ++b) {
            const uint16_t *blk = x + m * K + b * 16;
            double a = 0.0;
            unsigned sc, cd[16];
            for (int i = 0; i < 16; ++i) {
                double v = fabs(oracle_bf16_value(blk[i]));
                if (v > a || isnan(v))   /* a NaN stays the maximum */
                    a = v;
            }
            sc = oracle_scale_code(a);
            scales[m * (K / 16) + b] = (uint8_t)sc;
            for (int i = 0; i < 16; ++i)
                cd[i] = oracle_e2m1_encode(blk[i], sc);
            for (int j = 0; j < 8; ++j)
                codes[m * (K / 2) + b * 8 + j] = (uint8_t)(cd[2 * j] | (cd[2 * j + 1] << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Two-level NVFP4: a per-tensor fp32 scale above the per-16 E4M3 scales       */
/* ------------------------------------------------------------------------ */

/* The deployed NVFP4 checkpoints come from NVFP4 quantization tools [P4
 * section 1 and its sources: NVIDIA ModelOpt NVFP4 checkpoints]; the pages do
 * not spell out their scaling.  Readings taken (the plainest that keeps the
 * per-16 rule above unchanged):
 *   - a tensor carries one positive fp32 global scale g, and an element is
 *     e2m1(code) * e4m3(scale) * g;
 *   - the offline quantizer picks g = fl32(amax / 2688), 2688 = 6 * 448 (the
 *     largest e2m1 magnitude times the largest E4M3 scale), so the block
 *     holding the tensor's amax gets scale 448; an all-zero tensor takes g = 1;
 *   - every element is first divided by g in binary32, y = fl32(x / g), and
 *     the single-level rule (scale from the block's max |y| / 6, codes against
 *     it) is applied to y unchanged. */
float oracle_global_scale(double amax)
{
    return amax > 0.0 ? (float)(amax / 2688.0) : 1.0f;
}

/* Quantize bf16 rows x [M][K] with a given global scale g (> 0): codes
 * [M][K/2], scales [M][K/16] of y = fl32(x / g).  g = 1 gives exactly
 * oracle_quantize. */
void oracle_quantize_scaled(const uint16_t *x, int64_t M, int64_t K, float g, uint8_t *codes,
                            uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < K / 16; ++b) {
            double y[16], a = 0.0, s;
            unsigned sc, cd[16];
            for (int i = 0; i < 16; ++i) {
                /* binary32 quotient: the double quotient rounded to binary32 */
                y[i] = (double)(float)(oracle_bf16_value(x[m * K + b * 16 + i]) / (double)g);
                if (fabs(y[i]) > a || isnan(y[i]))   /* a NaN stays the maximum */
                    a = fabs(y[i]);
            }
            sc = oracle_scale_code(a);
            s = oracle_e4m3_value(sc);
            scales[m * (K / 16) + b] = (uint8_t)sc;
            for (int i = 0; i < 16; ++i) {
                unsigned mag = (s == 0.0) ? 0u : oracle_e2m1_index(fabs(y[i]), s);
                cd[i] = ((signbit(y[i]) ? 1u : 0u) << 3) | mag;
            }
            for (int j = 0; j < 8; ++j)
                codes[m * (K / 2) + b * 8 + j] = (uint8_t)(cd[2 * j] | (cd[2 * j + 1] << 4));
        }
    }
}

/* Offline weight quantizer: bf16 weights w [N][K] -> two-level NVFP4 (codes,
 * scales, returned g).  g comes from the whole tensor's max |w|. */
float oracle_quantize_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                             uint8_t *scales)
{
    double amax = 0.0;
    float g;
    for (int64_t i = 0; i < N * K; ++i) {
        double v = fabs(oracle_bf16_value(w[i]));
        if (v > amax)
            amax = v;
    }
    g = oracle_global_scale(amax);
    oracle_quantize_scaled(w, N, K, g, codes, scales);
    return g;
}

/* Dequantize a two-level NVFP4 matrix to bf16: the exact value
 * e2m1 * e4m3 * g rounded to binary32, then to bf16 (nearest even both). */
void oracle_dequantize_scaled(const uint8_t *codes, const uint8_t *scales, float g, int64_t N,
                              int64_t K, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_e2m1_value(code_at(codes + n * (K / 2), k)) *
                       oracle_e4m3_value(scales[n * (K / 16) + k / 16]) * (double)g;
            out[n * K + k] = oracle_bf16_round((double)(float)v);
        }
}

/* ------------------------------------------------------------------------ */
/* Contractions                                                               */
/* ------------------------------------------------------------------------ */

static void dequant_row_f64(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t n,
                            double *w)
{
    const uint8_t *rc = codes + n * (K / 2);
    const uint8_t *rs = scales + n * (K / 16);
    for (int64_t k = 0; k < K; ++k)
        w[k] = oracle_e2m1_value(code_at(rc, k)) * oracle_e4m3_value(rs[k / 16]);
}

/* W4A16 linear layer [P4 section 1; P3 "What the artifact is"]:
 *   out[m][j] = sum_k x[m][k] * w[n_j][k],  n_j = row_idx ? row_idx[j] : j,
 * with w the dequantized NVFP4 weight (nn.Linear orientation, y = x W^T).
 * Every product is exact in double and the sum runs over k in order in fp64.
 * row_idx selects a subset of weight rows [P3 "The masked head trick"]; the
 * output is compact [M][n_out] in row_idx order.  out is fp64 (unrounded). */
void oracle_gemm_w4a16(const uint16_t *x, int64_t M, int64_t K, const uint8_t *w_codes,
                       const uint8_t *w_scales, const int32_t *row_idx, int64_t n_out,
                       double *out)
{
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < n_out; ++j) {
            int64_t n = row_idx ? (int64_t)row_idx[j] : j;
            dequant_row_f64(w_codes, w_scales, K, n, w);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += oracle_bf16_value(x[m * K + k]) * w[k];
                out[m * n_out + j] = acc;
            }
        }
        free(w);
    }
}

/* W4A4 linear layer [P1]: both operands NVFP4.  A is dequantized to bf16 (the
 * dequantized value is exact in bf16) and the W4A16 definition is applied. */
void oracle_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                      const uint8_t *w_codes, const uint8_t *w_scales, const int32_t *row_idx,
                      int64_t n_out, double *out)
{
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * K));
    oracle_dequantize(a_codes, a_scales, M, K, a);
    oracle_gemm_w4a16(a, M, K, w_codes, w_scales, row_idx, n_out, out);
    free(a);
}

/* ------------------------------------------------------------------------ */
/* Routed mixture of experts [P4 section 1: a routed-expert layer; section 7:  */
/* NVFP4 expert weights executed by a grouped kernel]                          */
/* ------------------------------------------------------------------------ */

/* Routing preparation: a stable counting sort of the T*topk (token, slot)
 * assignments by expert.  Assignment p = t*topk + j goes to expert ids[p].
 *   offsets[e] .. offsets[e+1]-1 : the rows of expert e (offsets[E] = T*topk),
 *   gather_idx[r]               : the token whose activation row r reads,
 *   slot_pos[p]                 : the row r that assignment p landed in.
 * Within an expert, rows keep ascending p.  Returns 0, or -1 if an id is out
 * of range. */
int oracle_moe_align(const int32_t *ids, int64_t T, int64_t topk, int64_t E, int32_t *offsets,
                     int32_t *gather_idx, int32_t *slot_pos)
{
    int64_t R = T * topk;
    int64_t *fill = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t e = 0; e <= E; ++e)
        offsets[e] = 0;
    for (int64_t p = 0; p < R; ++p) {
        if (ids[p] < 0 || ids[p] >= E) {
            free(fill);
            return -1;
        }
        offsets[ids[p] + 1] += 1;
    }
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];
    for (int64_t p = 0; p < R; ++p) {
        int64_t e = ids[p];
        int64_t r = offsets[e] + fill[e]++;
        gather_idx[r] = (int32_t)(p / topk);
        slot_pos[p] = (int32_t)r;
    }
    free(fill);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Grouped W4A16 GEMM over experts.  Row r (0 <= r < R) belongs to the expert
 * e with offsets[e] <= r < offsets[e+1]; it reads activation row
 * src = gather_idx ? gather_idx[r] : r of a (bf16 [a_rows][K]) and computes
 *   h[n] = sum_k a[src][k] * w_e[n][k]  (fp64, n < N)
 * with w_e the dequantized weights of expert e (codes [E][N][K/2], scales
 * [E][N][K/16]).  Epilogue:
 *   epi == 0: out[r][n] = h[n]
 *   epi == 1 (gated, reading of a fused gate+up weight: first half of the
 *            rows is the gate, second half the up projection):
 *            out[r][i] = silu(h[i]) * h[i + N/2],  i < N/2
 * Two-level weights (reading of [P4] section 1: the deployed MoE checkpoints
 * come from NVFP4 quantization tools, whose tensors carry one fp32 global
 * scale each): if w_global (fp32 [E]) is given, every h[n] of expert e is
 * multiplied by w_global[e] before the epilogue (the gate and up halves of a
 * fused W1 share their expert's scale).
 * Then, if row_scale, out[r][.] *= row_scale[r].  out is fp64 (unrounded),
 * width N or N/2. */
void oracle_grouped_gemm(const uint16_t *a, int64_t K, const int32_t *gather_idx,
                         const int32_t *offsets, int64_t E, int64_t R, int64_t N,
                         const uint8_t *w_codes, const uint8_t *w_scales, const float *w_global,
                         const float *row_scale, int epi, double *out)
{
    int64_t width = (epi == 1) ? N / 2 : N;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t e = 0; e < E; ++e) {
            const uint8_t *ce = w_codes + e * N * (K / 2);
            const uint8_t *se = w_scales + e * N * (K / 16);
            double ge = w_global ? (double)w_global[e] : 1.0;
            for (int64_t r = offsets[e]; r < offsets[e + 1] && r < R; ++r) {
                int64_t src = gather_idx ? (int64_t)gather_idx[r] : r;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    dequant_row_f64(ce, se, K, n, w);
                    for (int64_t k = 0; k < K; ++k)
                        acc += oracle_bf16_value(a[src * K + k]) * w[k];
                    h[n] = acc * ge;
                }
                for (int64_t i = 0; i < width; ++i) {
                    double v = (epi == 1) ? silu(h[i]) * h[i + N / 2] : h[i];
                    if (row_scale)
                        v *= (double)row_scale[r];
                    out[r * width + i] = v;
                }
            }
        }
        free(w);
        free(h);
    }
}

/* Combine: out[t][c] = sum_{j < topk} y[slot_pos[t*topk + j]][c] in fp64, slot
 * order; y is bf16 [R][H]; out fp64 [T][H]. */
void oracle_moe_combine(const uint16_t *y, const int32_t *slot_pos, int64_t T, int64_t topk,
                        int64_t H, double *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < topk; ++j)
                acc += oracle_bf16_value(y[(int64_t)slot_pos[t * topk + j] * H + c]);
            out[t * H + c] = acc;
        }
}

/* The whole routed-expert layer, token by token (no sorting, no grouping):
 * for token t and slot j, with e = ids[t][j] and gate g = gates[t][j],
 *   h   = x[t] . W1_e^T                      (fp64, 2I values)
 *   act = bf16( silu(h[0:I]) * h[I:2I] )     (stored between the two GEMMs)
 *   y_j = bf16( g * (act . W2_e^T) )         (stored per slot)
 *   out[t] = sum_j y_j                       (fp64, slot order; unrounded)
 * W1: codes [E][2I][H/2], scales [E][2I][H/16]; W2: codes [E][H][I/2], scales
 * [E][H][I/16].  Two-level weights: w1_global / w2_global (fp32 [E], or NULL
 * for 1) multiply h and act . W2_e^T of expert e (as in oracle_grouped_gemm).
 * The bf16 rounding points are where this library stores intermediates in
 * bf16. */
void oracle_moe_layer(const uint16_t *x, int64_t T, int64_t H, const int32_t *ids,
                      const float *gates, int64_t topk, int64_t E, int64_t I,
                      const uint8_t *w1_codes, const uint8_t *w1_scales,
                      const uint8_t *w2_codes, const uint8_t *w2_scales,
                      const float *w1_global, const float *w2_global, double *out)
{
    (void)E;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
        double *acc = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t c = 0; c < H; ++c)
                acc[c] = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                int64_t e = ids[t * topk + j];
                double g = (double)gates[t * topk + j];
                double g1 = w1_global ? (double)w1_global[e] : 1.0;
                double g2 = w2_global ? (double)w2_global[e] : 1.0;
                const uint8_t *c1 = w1_codes + e * (2 * I) * (H / 2);
                const uint8_t *s1 = w1_scales + e * (2 * I) * (H / 16);
                const uint8_t *c2 = w2_codes + e * H * (I / 2);
                const uint8_t *s2 = w2_scales + e * H * (I / 16);
                for (int64_t n = 0; n < 2 * I; ++n) {
                    double s = 0.0;
                    dequant_row_f64(c1, s1, H, n, w);
                    for (int64_t k = 0; k < H; ++k)
                        s += oracle_bf16_value(x[t * H + k]) * w[k];
                    h[n] = s * g1;
                }
                for (int64_t i = 0; i < I; ++i)
                    act[i] = oracle_bf16_value(oracle_bf16_round(silu(h[i]) * h[i + I]));
                for (int64_t c = 0; c < H; ++c) {
                    double s = 0.0;
                    dequant_row_f64(c2, s2, I, c, w);
                    for (int64_t k = 0; k < I; ++k)
                        s += act[k] * w[k];
                    acc[c] += oracle_bf16_value(oracle_bf16_round(g * (s * g2)));
                }
            }
            for (int64_t c = 0; c < H; ++c)
                out[t * H + c] = acc[c];
        }
        free(w);
        free(h);
        free(act);
        free(acc);
    }
}

/* ------------------------------------------------------------------------ */
/* Draft proposal from the masked head                                        */
/* ------------------------------------------------------------------------ */

/* Order of two head outputs for the draft proposal: the larger logit first.
 * Readings (the pages only say that the draft proposes tokens from the
 * masked head [P3 "The masked head trick"]): equal logits rank the smaller
 * column first (the column is the position in the ranked mask, so the more
 * frequent token wins), and -0 ranks below +0 (the order of the fp32 bit
 * patterns).  NaN is outside the contract. */
typedef struct {
    double v;
    int64_t col;
} topk_item;

static int topk_before(const void *pa, const void *pb)
{
    const topk_item *a = (const topk_item *)pa, *b = (const topk_item *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    if (signbit(a->v) != signbit(b->v)) return signbit(a->v) ? 1 : -1;
    if (a->col < b->col) return -1;
    if (a->col > b->col) return 1;
    return 0;
}

/* Top-k of each row of v [M][n] under the order above, best first:
 * out_v[m][i] is the i-th best value, out_ids[m][i] its vocabulary id
 * (ids_map[col] when the columns are a masked subset, else col).  A full
 * sort per row; k <= n. */
void oracle_topk(const double *v, int64_t M, int64_t n, int64_t k, const int32_t *ids_map,
                 double *out_v, int32_t *out_ids)
{
#pragma omp parallel
    {
        topk_item *items = (topk_item *)malloc(sizeof(topk_item) * (size_t)n);
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t c = 0; c < n; ++c) {
                items[c].v = v[m * n + c];
                items[c].col = c;
            }
            qsort(items, (size_t)n, sizeof(topk_item), topk_before);
            for (int64_t i = 0; i < k; ++i) {
                out_v[m * k + i] = items[i].v;
                out_ids[m * k + i] =
                    ids_map ? ids_map[items[i].col] : (int32_t)items[i].col;
            }
        }
        free(items);
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 KV-cache codec                                                    */
/* ------------------------------------------------------------------------ */

/* E4M3 code of a real value v [P4 section 3: the KV cache stored as FP8
 * E4M3].  Readings: round to the nearest E4M3 value, ties to the even code;
 * magnitudes at or above 448 saturate to 448 (satfinite: there is no
 * infinity); the sign is kept, zero included; a NaN becomes the NaN code of
 * its sign (the format's only non-finite codes, 0x7F and 0xFF).  Written as
 * the plain nearest search over the 127 non-negative finite values; every
 * comparison is exact
 * in double (E4M3 values and their midpoints have at most 5 significant
 * bits). */
unsigned oracle_e4m3_encode(double v)
{
    unsigned sign = signbit(v) ? 0x80u : 0u;
    double a = fabs(v);
    unsigned c = 0;
    if (isnan(v))
        return sign | 0x7Fu;              /* NaN keeps its sign: code 0x7F / 0xFF */
    for (unsigned cand = 1; cand <= 0x7E; ++cand)
        if (oracle_e4m3_value(cand) <= a)
            c = cand;
    if (c < 0x7E) {
        double mid = 0.5 * (oracle_e4m3_value(c) + oracle_e4m3_value(c + 1));
        if (a > mid || (a == mid && ((c + 1) & 1u) == 0))
            c = c + 1;
    }
    return sign | c;
}

/* Quotient x / scale rounded once to binary32 (nearest even).  The double
 * quotient is rounded to 53 bits first; for a division that second rounding
 * cannot change the binary32 result (53 >= 2*24 + 2). */
static double f32_quotient(double x, double scale)
{
    return (double)(float)(x / scale);
}

/* Store tokens into an FP8 E4M3 KV cache [P4 section 3: FP8 E4M3 KV cache,
 * 16-token pages by default].  x is bf16 [T][W] (W = heads * head size of
 * one of K or V); cache is [num_slots][W] codes, where a slot is
 * page * page_size + position in the page, so the paged layout
 * [pages][page_size][W] is this array.  Reading (the pages give no scale
 * rule): one positive fp32 scale per cache, code = E4M3(fl32(x / scale)).
 * slot_mapping[t] < 0 (padding) or >= num_slots leaves the cache untouched. */
void oracle_kv_store_e4m3(const uint16_t *x, int64_t T, int64_t W, const int32_t *slot_mapping,
                          float scale, uint8_t *cache, int64_t num_slots)
{
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        for (int64_t w = 0; w < W; ++w)
            cache[slot * W + w] = (uint8_t)oracle_e4m3_encode(
                f32_quotient(oracle_bf16_value(x[t * W + w]), (double)scale));
    }
}

/* Read B sequences back from the cache: out bf16 [B][max_len][W],
 *   out[b][i][w] = bf16(fl32(e4m3(cache[s][w]) * scale)),
 *   s = block_table[b][i / page_size] * page_size + i % page_size,
 * for i < seq_lens[b]; zero for i >= seq_lens[b] and for a slot outside the
 * cache.  The product is formed exactly, rounded to binary32, then to bf16
 * (both nearest even): dequantize in fp32, store bf16. */
void oracle_kv_load_e4m3(const uint8_t *cache, int64_t num_slots, int64_t W,
                         const int32_t *block_table, const int32_t *seq_lens, int64_t B,
                         int64_t max_pages, int64_t page_size, int64_t max_len, float scale,
                         uint16_t *out)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < max_len; ++i) {
            uint16_t *o = out + (b * max_len + i) * W;
            int64_t slot = -1;
            if (i < seq_lens[b] && i / page_size < max_pages) {
                int64_t page = block_table[b * max_pages + i / page_size];
                slot = page * page_size + i % page_size;
            }
            if (slot < 0 || slot >= num_slots) {
                for (int64_t w = 0; w < W; ++w)
                    o[w] = 0;
                continue;
            }
            for (int64_t w = 0; w < W; ++w) {
                double p = oracle_e4m3_value(cache[slot * W + w]) * (double)scale;
                o[w] = oracle_bf16_round((double)(float)p);
            }
        }
}

/* Number of threads the parallel loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
