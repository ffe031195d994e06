"""GPU parity of two-level NVFP4 (per-tensor fp32 scale) against the oracle:
the offline weight quantizer, the activation quantizer with a given scale and
the scaled dequantization are bit-exact; scaled GEMMs meet the GEMM tolerance
(relative Frobenius error <= 1e-3, every element within 1e-2*(|ref|+1))."""
import numpy as np
import pytest

import helpers
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available()
    import bit_quantized_gemm_nvfp4_amd as m
    m.lib()
    return m


def _weights(seed, N, K):
    """Rows of very different magnitude (2^-12 .. 2^3 times N(0,1)), like the
    layers of a trained checkpoint."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, K)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-12, 4, size=(N, 1)).astype(np.float32)
    return workloads.f32_to_bf16_bits(x)


def _g(t):
    return float(t.cpu().numpy()[0])


@pytest.mark.parametrize("N,K,seed", [(1, 32, 0), (37, 96, 1), (300, 512, 2), (64, 2048, 3)])
def test_quantize_weight_bit_exact(nv, orc, N, K, seed):
    helpers.announce(f"quantize_weight N={N} K={K}")
    w = _weights(seed, N, K)
    c, s, g = nv.quantize_weight(helpers.dev_bf16(w))
    oc, os_, og = orc.quantize_weight(w, N, K)
    assert _g(g) == og
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)


def test_quantize_weight_all_zero(nv, orc):
    helpers.announce("quantize_weight zeros")
    w = np.zeros((8, 64), dtype=np.uint16)
    w[::2, ::3] = 0x8000                                   # negative zeros keep their sign bit
    c, s, g = nv.quantize_weight(helpers.dev_bf16(w))
    oc, os_, og = orc.quantize_weight(w, 8, 64)
    assert _g(g) == og == 1.0
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)


def test_quantize_weight_full_size_sampled(nv, orc):
    """K=5120 -> N=17408 weights: the global scale matches, and 256 sampled rows
    match the oracle's rows quantized with that scale."""
    helpers.announce("quantize_weight N=17408 K=5120")
    N, K = workloads.MLP, workloads.HIDDEN
    w = _weights(4, N, K)
    c, s, g = nv.quantize_weight(helpers.dev_bf16(w))
    amax = float(np.abs(helpers.bf16_bits_to_f64(w)).max())
    og = orc.global_scale(amax)
    assert _g(g) == og
    rows = np.sort(np.random.default_rng(5).choice(N, 256, replace=False))
    oc, os_ = orc.quantize_scaled(w[rows], 256, K, og)
    assert np.array_equal(c.cpu().numpy()[rows], oc)
    assert np.array_equal(s.cpu().numpy()[rows], os_)


@pytest.mark.parametrize("gval", [1.0, 0.0123, 3.75, 2.0 ** -30])
def test_quantize_scaled_bit_exact(nv, orc, gval):
    import torch
    helpers.announce(f"quantize_scaled M=512 K=5120 g={gval}")
    x = workloads.normal_bf16(np.random.default_rng(6), 512, 5120, outlier_frac=0.001)
    g = torch.tensor([gval], dtype=torch.float32, device="cuda")
    c, s = nv.quantize_scaled(helpers.dev_bf16(x), g)
    oc, os_ = orc.quantize_scaled(x, 512, 5120, gval)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    if gval == 1.0:  # the single-level quantizer
        c1, s1 = nv.quantize(helpers.dev_bf16(x))
        assert torch.equal(c1, c) and torch.equal(s1, s)


def test_dequantize_scaled_bit_exact(nv, orc):
    import torch
    helpers.announce("dequantize_scaled N=300 K=512")
    w = workloads.nvfp4_weight(np.random.default_rng(7), 300, 512)
    for gval in (1.0, 0.00731, 113.0):
        g = torch.tensor([gval], dtype=torch.float32, device="cuda")
        got = helpers.host_bits(nv.dequantize_scaled(helpers.dev_u8(w.codes),
                                                     helpers.dev_u8(w.scales), g))
        assert np.array_equal(got, orc.dequantize_scaled(w.codes, w.scales, gval, 300, 512))


@pytest.mark.parametrize("M,K,N", [(1, 512, 1024), (8, 5120, 1000), (32, 1024, 300),
                                   (300, 512, 520), (70, 4096, 256)])
def test_gemm_scaled_w4a16(nv, orc, M, K, N):
    """bf16 weights quantized on the GPU, then the scaled product; M >= 65 takes
    the MFMA GEMM (K=4096, N=256 also splits K)."""
    import torch
    helpers.announce(f"gemm_scaled w4a16 M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    wb = _weights(M + N, N, K)
    x = workloads.normal_bf16(rng, M, K)
    c, s, g = nv.quantize_weight(helpers.dev_bf16(wb))
    y = helpers.host_bits(nv.gemm_scaled(helpers.dev_bf16(x), c, s, w_global_scale=g))
    oc, os_, og = orc.quantize_weight(wb, N, K)
    ref = orc.gemm_scaled(x, M, K, oc, os_, og)
    ok, rf, worst = helpers.gemm_close(y, ref)
    assert ok, f"rel_frob={rf:.3e} worst={worst:.3f}"
    # unscaled entry point on the same codes: the scaled result is that times g
    y1 = nv.gemm(helpers.dev_bf16(x), c, s, out_dtype=torch.float32)
    y2 = nv.gemm_scaled(helpers.dev_bf16(x), c, s, w_global_scale=g, out_dtype=torch.float32)
    assert torch.equal(y2, y1 * g[0])


@pytest.mark.parametrize("M", [16, 512])
def test_gemm_scaled_w4a4(nv, orc, M):
    """Two-level activations (static scale) and weights (offline quantizer)."""
    import torch
    helpers.announce(f"gemm_scaled w4a4 M={M}")
    K, N = 1024, 768
    x = workloads.normal_bf16(np.random.default_rng(8), M, K, outlier_frac=0.001)
    wb = _weights(9, N, K)
    ga = torch.tensor([0.0057], dtype=torch.float32, device="cuda")
    ac, as_ = nv.quantize_scaled(helpers.dev_bf16(x), ga)
    c, s, g = nv.quantize_weight(helpers.dev_bf16(wb))
    y = helpers.host_bits(nv.gemm_scaled(ac, c, s, w_global_scale=g, a_scales=as_,
                                         a_global_scale=ga))
    oac, oas = orc.quantize_scaled(x, M, K, 0.0057)
    oc, os_, og = orc.quantize_weight(wb, N, K)
    ref = orc.gemm_scaled(oac, M, K, oc, os_, og, a_scales=oas, a_g=float(np.float32(0.0057)))
    ok, rf, worst = helpers.gemm_close(y, ref)
    assert ok, f"rel_frob={rf:.3e} worst={worst:.3f}"
