"""Pins of the oracle's two-level NVFP4 (per-tensor fp32 scale) and offline
weight quantizer: the g = 1 case is the single-level quantizer; power-of-two
rescaling of the weights leaves codes and scales unchanged and rescales g; the
tensor's amax block gets scale 448; g against numpy's binary32 division; block
scales against torch's float8 cast and codes against a brute-force nearest
search (numpy); dequantization against numpy's binary32 products and torch's
bf16 cast; the scaled product against numpy BLAS."""
import numpy as np
import torch

import helpers
import workloads


def _weights(seed, N, K, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, K)).astype(np.float32)
    if spread:  # rows of very different magnitude, like a trained layer
        x *= np.float32(2.0) ** rng.integers(-12, 4, size=(N, 1)).astype(np.float32)
    return workloads.f32_to_bf16_bits(x)


def test_unit_global_scale_is_single_level(orc):
    x = workloads.normal_bf16(np.random.default_rng(40), 24, 256, outlier_frac=0.01)
    c1, s1 = orc.quantize(x, 24, 256)
    c2, s2 = orc.quantize_scaled(x, 24, 256, 1.0)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_power_of_two_rescaling_invariance(orc):
    w = _weights(41, 32, 128)
    c, s, g = orc.quantize_weight(w, 32, 128)
    for j in (-3, 5):
        wj = helpers.f64_to_bf16_bits_exact(helpers.bf16_bits_to_f64(w) * 2.0 ** j)
        cj, sj, gj = orc.quantize_weight(wj, 32, 128)
        assert np.array_equal(cj, c) and np.array_equal(sj, s)
        assert gj == g * 2.0 ** j


def test_global_scale_and_amax_block(orc):
    w = _weights(42, 16, 96)
    a = np.abs(helpers.bf16_bits_to_f64(w))
    c, s, g = orc.quantize_weight(w, 16, 96)
    assert g == float(np.float32(a.max()) / np.float32(2688.0))
    r, k = np.unravel_index(np.argmax(a), a.shape)
    assert s[r, k // 16] == 0x7E
    z = np.zeros((4, 32), dtype=np.uint16)
    cz, sz, gz = orc.quantize_weight(z, 4, 32)
    assert gz == 1.0 and not cz.any() and not sz.any()


def _torch_e4m3(v32):
    v = np.ascontiguousarray(v32, dtype=np.float32)
    sat = v > 448.0
    codes = torch.from_numpy(np.where(sat, 0.0, v).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes[sat] = 0x7E
    return codes


def test_scales_and_codes_brute_force(orc):
    N, K = 20, 160
    w = _weights(43, N, K)
    c, s, g = orc.quantize_weight(w, N, K)
    y = (helpers.bf16_bits_to_f64(w).astype(np.float32) / np.float32(g)).astype(np.float64)
    yb = y.reshape(N, K // 16, 16)
    amax = np.abs(yb).max(axis=2)
    want_s = _torch_e4m3(amax.astype(np.float32) / np.float32(6.0))
    assert np.array_equal(s, want_s)
    sv = helpers.e4m3_table_torch()[s][:, :, None]
    mags = np.abs(helpers.e2m1_table()[:8])                       # 0, .5, 1, 1.5, 2, 3, 4, 6
    d = np.abs(np.abs(yb)[..., None] - sv[..., None] * mags)     # exact in fp64
    best = d.min(axis=-1, keepdims=True)
    tie_even = np.where(d == best, np.arange(8) % 2 == 0, False).any(axis=-1)
    idx = np.where(tie_even,
                   np.argmax((d == best) & (np.arange(8) % 2 == 0), axis=-1),
                   np.argmax(d == best, axis=-1))
    idx = np.where(sv == 0, 0, idx)
    code = idx | (np.signbit(yb).astype(np.int64) << 3)
    lo, hi = c & 15, c >> 4
    got = np.stack([lo, hi], axis=-1).reshape(N, K // 16, 16)
    assert np.array_equal(got, code)


def test_dequantize_scaled_matches_numpy_and_torch(orc):
    N, K = 12, 64
    w = workloads.nvfp4_weight(np.random.default_rng(44), N, K)
    g = 0.00123
    got = orc.dequantize_scaled(w.codes, w.scales, g, N, K)
    v32 = helpers.dequant_independent(w.codes, w.scales).astype(np.float32) * np.float32(g)
    want = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_round_trip_error_within_half_step(orc):
    N, K = 16, 256
    w = _weights(45, N, K)
    c, s, g = orc.quantize_weight(w, N, K)
    back = helpers.dequant_independent(c, s)                       # e2m1 * e4m3, exact
    y = helpers.bf16_bits_to_f64(w).astype(np.float32).astype(np.float64) / g
    sv = np.repeat(helpers.e4m3_table_torch()[s], 16, axis=1)
    assert np.all(np.abs(back - y) <= sv * 1.0 + np.abs(y) * 2.0 ** -22)


def test_scaled_gemm_matches_blas(orc):
    rng = np.random.default_rng(46)
    M, N, K = 8, 48, 128
    x = workloads.normal_bf16(rng, M, K)
    wb = _weights(47, N, K)
    c, s, g = orc.quantize_weight(wb, N, K)
    got = orc.gemm_scaled(x, M, K, c, s, g)
    W = helpers.dequant_independent(c, s) * g
    ref = helpers.bf16_bits_to_f64(x) @ W.T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
