"""Pins of the oracle's contractions: closed forms, brute force with exact
rational arithmetic on tiny shapes, and numpy fp64 BLAS (a library routine) on
weights dequantized by an independent decoder."""
from fractions import Fraction

import numpy as np

import helpers
import workloads


def _parse_closed_forms():
    for line in helpers.golden_lines("gemm_closed_forms.txt"):
        name, K, xrule, crule, sc, y = [p.strip() for p in line.split("|")]
        yield name, int(K), xrule, [int(b, 16) for b in crule.split()], int(sc, 16), float(y)


def test_gemm_closed_forms(orc):
    e2m1 = helpers.e2m1_table()
    for name, K, xrule, cbytes, sc, y in _parse_closed_forms():
        codes = np.resize(np.array(cbytes, np.uint8), K // 2).reshape(1, K // 2)
        scales = np.full((1, K // 16), sc, np.uint8)
        if xrule == "ones":
            xv = np.ones(K)
        else:  # the e2m1 values of the codes, in element order
            el = np.stack([codes[0] & 15, codes[0] >> 4], axis=1).reshape(-1)
            xv = e2m1[el]
        x = helpers.f64_to_bf16_bits_exact(xv).reshape(1, K)
        got = orc.gemm_w4a16(x, 1, K, codes, scales)
        assert got[0, 0] == y, (name, got[0, 0], y)


def test_gemm_brute_force_exact_tiny(orc):
    """M=3, N=5, K=64 with exact Fraction arithmetic: the fp64 oracle sum of exact
    products must equal the exact rational sum to within fp64 rounding."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 5, 64
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    got = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    e2m1 = [Fraction(float(v)) for v in helpers.e2m1_table()]
    e4m3 = helpers.e4m3_table_torch()
    xv = helpers.bf16_bits_to_f64(x)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                byte = int(w.codes[n, k // 2])
                c = (byte >> 4) if k % 2 else (byte & 15)
                term = Fraction(float(xv[m, k])) * e2m1[c] * Fraction(float(e4m3[w.scales[n, k // 16]]))
                acc += term
                mag += abs(term)
            assert abs(Fraction(got[m, n]) - acc) <= mag * Fraction(1, 2**50), (m, n)


def test_gemm_matches_numpy_blas(orc):
    rng = np.random.default_rng(6)
    M, N, K = 8, 96, 512
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    got = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    W = helpers.dequant_independent(w.codes, w.scales)
    ref = helpers.bf16_bits_to_f64(x) @ W.T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_dequantize_matches_independent_decoder(orc):
    """Oracle dequant (bf16 bits) vs table lookup through torch's E4M3 decode; the
    product is exact so the comparison is exact, sign of zero included.  Rows 0..255
    pair every code byte with scale code r (zero, negative and NaN scales too);
    the rest are random weights."""
    rng = np.random.default_rng(7)
    K = 512
    w = workloads.nvfp4_weight(rng, 64, K)
    all_bytes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scale_rows = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    codes = np.concatenate([all_bytes, w.codes], axis=0)
    scales = np.concatenate([scale_rows, w.scales], axis=0)
    N = codes.shape[0]
    got = helpers.bf16_bits_to_f64(orc.dequantize(codes, scales, N, K))
    ref = helpers.dequant_independent(codes, scales)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_masked_gemm_is_row_gather(orc):
    rng = np.random.default_rng(8)
    M, N, K = 4, 300, 256
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, 77, replace=False)).astype(np.int32)
    full = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    part = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx)
    assert np.array_equal(part, full[:, idx])


def test_masked_head_ratio_matches_page():
    """The masked head keeps 32,768 of 248,320 rows: the weight bytes streamed
    shrink by 248320/32768 = 7.58, printed on the page as 7.6x."""
    vals = dict(line.split() for line in helpers.golden_lines("masked_head.txt"))
    assert workloads.VOCAB == int(vals["vocab_rows"])
    assert workloads.MASKED_ROWS == int(vals["kept_rows"])
    full = workloads.VOCAB * workloads.HIDDEN * 9 // 16
    kept = workloads.MASKED_ROWS * workloads.HIDDEN * 9 // 16
    assert round(full / kept, 1) == float(vals["read_shrink_rounded"])


def test_w4a4_matches_blas_on_dequantized_operands(orc):
    rng = np.random.default_rng(9)
    M, N, K = 16, 64, 256
    x = workloads.normal_bf16(rng, M, K, outlier_frac=0.01)
    w = workloads.nvfp4_weight(rng, N, K)
    ac, as_ = orc.quantize(x, M, K)
    got = orc.gemm_w4a4(ac, as_, M, K, w.codes, w.scales)
    A = helpers.dequant_independent(ac, as_)
    W = helpers.dequant_independent(w.codes, w.scales)
    ref = A @ W.T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gemm_tolerance_helper_detects_errors(orc):
    """The parity check used for GPU results: an exact result passes; a result with
    one transposed pair of columns or a dropped k-term fails."""
    rng = np.random.default_rng(10)
    M, N, K = 4, 64, 512
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    ok, rf, worst = helpers.gemm_close(orc.bf16_round(ref), ref)
    assert ok and rf == 0.0
    bad = ref.copy()
    bad[:, [3, 4]] = bad[:, [4, 3]]
    assert not helpers.gemm_close(orc.bf16_round(bad), ref)[0]
    W = helpers.dequant_independent(w.codes, w.scales)
    drop = ref - helpers.bf16_bits_to_f64(x)[:, 100:101] * W[:, 100][None, :]
    assert not helpers.gemm_close(orc.bf16_round(drop), ref)[0]
