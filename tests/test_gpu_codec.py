"""GPU parity of dequantize and quantize against the oracle: bit-exact."""
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


def test_dequantize_every_code_every_scale(nv, orc):
    """256 rows: row r pairs all 256 code bytes with scale code r (including zero,
    negative and NaN scales), then random rows with a ragged row count."""
    helpers.announce("dequantize: all code bytes x all scale codes")
    K = 512
    all_bytes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scale_rows = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    w = workloads.nvfp4_weight(np.random.default_rng(1), 37, K)
    codes = np.concatenate([all_bytes, w.codes])
    scales = np.concatenate([scale_rows, w.scales])
    N = codes.shape[0]
    got = helpers.host_bits(nv.dequantize(helpers.dev_u8(codes), helpers.dev_u8(scales)))
    ref = orc.dequantize(codes, scales, N, K)
    nan_ref = (ref & 0x7FFF) > 0x7F80
    nan_got = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_got, nan_ref)
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])


def test_dequantize_decode_weights(nv, orc):
    helpers.announce("dequantize: 17408x5120 decode weights, sampled rows")
    w = workloads.decode_weights(5120, 17408)
    got = nv.dequantize(helpers.dev_u8(w.codes), helpers.dev_u8(w.scales))
    rows = np.random.default_rng(2).choice(17408, 64, replace=False)
    ref = orc.dequantize(w.codes[rows], w.scales[rows], 64, 5120)
    assert np.array_equal(helpers.host_bits(got)[rows], ref)


def test_quantize_every_block_maximum(nv, orc):
    """One block per non-negative finite bf16 value a: [a, -a/2 ..] -- covers
    every scale rounding decision, including ties, subnormal scales and
    saturation."""
    helpers.announce("quantize: every bf16 block maximum")
    a = helpers.all_bf16_nonneg_finite()
    nb = len(a)
    blocks = np.zeros((nb, 32), np.uint16)
    blocks[:, 0] = a
    blocks[:, 1] = a | 0x8000
    av = helpers.bf16_bits_to_f64(a)
    half = orc.bf16_round(av / 2)
    blocks[:, 2] = half
    blocks[:, 3] = half | 0x8000
    blocks[:, 16] = a  # the second block of the row repeats the maximum
    x = helpers.dev_bf16(blocks)
    gc, gs = nv.quantize(x)
    rc, rs = orc.quantize(blocks, nb, 32)
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)


def test_quantize_every_value_against_every_scale(nv, orc):
    """For each positive finite scale code s, blocks with maximum 6*s (so the scale
    is exactly s) hold every bf16 x with |x| <= 6s, both signs: every code
    rounding decision of the quantizer."""
    helpers.announce("quantize: every value x every scale")
    pos = helpers.all_bf16_nonneg_finite()
    pv = helpers.bf16_bits_to_f64(pos)
    rows = []
    for sc in range(1, 0x7F):
        s = orc.e4m3_value(sc)
        amax_bits = helpers.f64_to_bf16_bits_exact([6.0 * s])[0]
        xs = pos[pv <= 6.0 * s]
        xs = np.concatenate([xs, xs | 0x8000])
        pad = (-len(xs)) % 15
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        blk = np.concatenate([np.full((xs.shape[0], 1), amax_bits, np.uint16), xs], axis=1)
        rows.append(blk)
    blocks = np.concatenate(rows)
    if blocks.shape[0] % 2:
        blocks = np.concatenate([blocks, np.zeros((1, 16), np.uint16)])
    x = blocks.reshape(-1, 32)
    M = x.shape[0]
    gc, gs = nv.quantize(helpers.dev_bf16(x))
    rc, rs = orc.quantize(x, M, 32)
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)


def test_quantize_w4a4_workload(nv, orc):
    """The W4A4 activations (512 x 5120, outlier channels): codes and scales
    bit-exact; then a ragged shape with rows of very different magnitudes."""
    helpers.announce("quantize: W4A4 activations 512x5120")
    x, _ = workloads.w4a4()
    gc, gs = nv.quantize(helpers.dev_bf16(x))
    rc, rs = orc.quantize(x, 512, 5120)
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)
    rng = np.random.default_rng(5)
    M, K = 37, 96
    v = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-130, 127, (M, 1)).clip(-126, 120)))
    xb = orc.bf16_round(v)
    xb[(xb & 0x7F80) == 0x7F80] = 0  # keep inputs finite
    gc, gs = nv.quantize(helpers.dev_bf16(xb))
    rc, rs = orc.quantize(xb, M, K)
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)


def test_quantize_nan_blocks_confined(nv, orc):
    """Blocks holding a NaN (outside the contract) take the NaN scale code and
    sign-only codes; every neighbouring block, scale byte and code byte is
    bit-exact against the oracle (nothing spills into the next byte)."""
    helpers.announce("quantize: NaN blocks confined")
    rng = np.random.default_rng(90)
    M, K = 6, 256
    x = workloads.normal_bf16(rng, M, K)
    x[0, 17] = 0x7FC0
    x[1, 0] = 0xFFC0
    x[2, 255] = 0x7F81          # a signalling-NaN pattern
    x[3, 40] = 0x7F80           # +inf: saturates
    x[4, 15], x[4, 16] = 0x7FC0, 0xFFC0   # NaNs in two neighbouring blocks
    gc, gs = nv.quantize(helpers.dev_bf16(x))
    rc, rs = orc.quantize(x, M, K)
    assert rs[0, 1] == 0x7F and rs[4, 0] == 0x7F and rs[4, 1] == 0x7F
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)
