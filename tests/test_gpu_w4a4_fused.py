"""GPU parity of the W4A4 product with the activation quantizer fused in
(nvfp4_gemm_w4a4_bf16): bit-identical to nvfp4_quantize followed by the W4A4
nvfp4_gemm on the GEMV (quantizer in the activation staging) and MFMA (quantize
then GEMM) paths, and within the GEMM tolerance of the oracle."""
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


def _x(rng, M, K):
    x = workloads.normal_bf16(rng, M, K, outlier_frac=0.01)
    x[0, :32] = 0                  # an all-zero block pair
    x[-1, 32:48] = 0x8000          # a block of negative zeros
    return x


# Up to (300, 1056) the quantizer launches take one lane per 8 elements;
# (1040, 4096) is past one round of the chip and takes the wider threads.
@pytest.mark.parametrize("M,K,N", [
    (1, 512, 1024), (3, 800, 333), (4, 5120, 4096), (5, 512, 1000), (8, 5120, 17408),
    (16, 800, 300), (17, 2048, 520), (32, 5120, 4000), (40, 1024, 777), (64, 512, 64),
    (65, 512, 300), (300, 1056, 520), (1040, 4096, 64),
])
def test_fused_equals_quantize_then_gemm(nv, M, K, N):
    import torch
    helpers.announce(f"w4a4 fused M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 131 + K + N)
    x = helpers.dev_bf16(_x(rng, M, K))
    w = workloads.nvfp4_weight(rng, N, K)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    for odt in (torch.float32, torch.bfloat16):
        fused = nv.gemm_w4a4(x, wc, ws, out_dtype=odt)
        ac, as_ = nv.quantize(x)
        ref = nv.gemm(ac, wc, ws, a_scales=as_, out_dtype=odt)
        assert torch.equal(fused.view(torch.int16) if odt == torch.bfloat16 else
                           fused.view(torch.int32),
                           ref.view(torch.int16) if odt == torch.bfloat16 else ref.view(torch.int32))


def test_fused_masked_rows_and_oracle(nv, orc):
    import torch
    helpers.announce("w4a4 fused masked M=8 K=5120")
    rng = np.random.default_rng(90)
    M, K, N = 8, 5120, 20000
    xb = _x(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, 3000, replace=False)).astype(np.int32)
    y = nv.gemm_w4a4(helpers.dev_bf16(xb), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                     row_idx=helpers.dev_i32(idx), out_dtype=torch.float32)
    ac, as_ = orc.quantize(xb, M, K)
    ref = orc.gemm_w4a4(ac, as_, M, K, w.codes, w.scales, row_idx=idx)
    ok, rf, worst = helpers.gemm_close(y.cpu().numpy(), ref, out_is_bf16=False)
    assert ok, f"rel_frob={rf:.3e} worst={worst:.3f}"


@pytest.mark.parametrize("M,K,N,plan", [(3, 1056, 700, None), (5, 512, 1000, None),
                                        (8, 5120, 4000, None), (6, 1312, 90000, None),
                                        (17, 2048, 520, None), (17, 2048, 520, "2,16"),
                                        (30, 1312, 700, "2,16")])
def test_fused_in_staging_forced(nv, M, K, N, plan):
    """The quantizer inside the GEMV's activation staging (whole-K staging for
    M <= 4, the streamed window for 5 <= M <= 8 and M > 8), forced for every
    shape (plan w4a4_fuse = 1): bit-identical to quantize then the W4A4 GEMM,
    including ragged K steps and split-K.  plan "2,16": two activation tiles
    in 16-wave workgroups (scale blocks when K % 256 == 0)."""
    import torch
    helpers.announce(f"w4a4 fused in staging M={M} K={K} N={N} plan={plan}")
    rng = np.random.default_rng(M * 17 + K + N)
    x = helpers.dev_bf16(_x(rng, M, K))
    w = workloads.nvfp4_weight(rng, N, K)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    pl = {"w4a4_fuse": 1}
    if plan:
        pl.update(gemv_tiles=int(plan.split(",")[0]), gemv_waves=int(plan.split(",")[1]))
    fused = nv.gemm_w4a4(x, wc, ws, out_dtype=torch.float32, plan=pl)
    ac, as_ = nv.quantize(x)
    ref = nv.gemm(ac, wc, ws, a_scales=as_, out_dtype=torch.float32)
    assert torch.equal(fused.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("M,K,N,fuse", [(65, 64, 16, 1), (300, 160, 520, 1), (300, 160, 520, 0),
                                        (700, 2048, 1000, 1), (512, 5120, 1100, 1),
                                        (1000, 2080, 300, 1)])
def test_mfma_fused_quantizer_tile_loads(nv, orc, M, K, N, fuse):
    """Large M: the quantizer inside the MFMA GEMM's activation tile loads
    (plan w4a4_fuse = 1), and the one-pass variant (0), against quantize then
    the W4A4 GEMM -- bit-identical (the same exact operands summed in the same
    order) -- and against the oracle within the GEMM tolerance.  Shapes with a
    partial last K step (K % 64 == 32), ragged M and N, outlier activations,
    and split-K tail tiles."""
    import torch
    helpers.announce(f"w4a4 mfma fused tile loads M={M} K={K} N={N} fuse={fuse}")
    rng = np.random.default_rng(M + 3 * K + N)
    xb = _x(rng, M, K)
    x = helpers.dev_bf16(xb)
    w = workloads.nvfp4_weight(rng, N, K)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    got = nv.gemm_w4a4(x, wc, ws, out_dtype=torch.float32, plan={"w4a4_fuse": fuse})
    ac, as_ = nv.quantize(x)
    ref = nv.gemm(ac, wc, ws, a_scales=as_, out_dtype=torch.float32)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    rc, rs = orc.quantize(xb, M, K)
    ok, rf, worst = helpers.gemm_close(got.cpu().numpy(),
                                       orc.gemm_w4a4(rc, rs, M, K, w.codes, w.scales),
                                       out_is_bf16=False)
    assert ok, f"rel_frob={rf:.3e} worst={worst:.3f}"
