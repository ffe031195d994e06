"""nvfp4_gemm_noalloc (the workspace in the library's device array) against
nvfp4_gemm (caller's workspace) through the C ABI: bit-identical outputs on
two calls in a row, the second smaller, and within the GEMM tolerance of the
oracle on sampled columns."""
import ctypes

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


def _noalloc(nv, a, a_scales, M, N, K, wc, ws, row_idx, n_out, out):
    import torch
    vp = ctypes.c_void_p
    st = vp(torch.cuda.current_stream().cuda_stream)
    rc = nv.lib().nvfp4_gemm_noalloc(nv.NVFP4 if a_scales is not None else nv.BF16,
                                     vp(a.data_ptr()),
                                     None if a_scales is None else vp(a_scales.data_ptr()),
                                     M, N, K, vp(wc.data_ptr()), vp(ws.data_ptr()),
                                     None if row_idx is None else vp(row_idx.data_ptr()), n_out,
                                     nv.BF16, vp(out.data_ptr()), st)
    assert rc == 0, nv.lib().nvfp4_status_string(rc)


# (M, K, N, masked rows, W4A4): split-K GEMV partials, a masked head-like call,
# MFMA split-K tail tiles, W4A4 with the dequantized activations in scratch
CASES = [
    [(32, 17408, 5120, 0, False), (8, 5120, 4000, 0, False)],
    [(32, 5120, 40000, 3000, False), (1, 2048, 3000, 0, False)],
    [(1300, 2560, 12797, 0, False), (300, 2080, 300, 0, False)],
    [(512, 1024, 3000, 0, True), (70, 512, 1000, 0, True)],
]


@pytest.mark.parametrize("pair", CASES)
def test_noalloc_matches_gemm_two_calls(nv, orc, pair):
    import torch
    for i, (M, K, N, n_mask, w4a4) in enumerate(pair):
        helpers.announce(f"gemm_noalloc call {i} M={M} K={K} N={N} mask={n_mask} w4a4={w4a4}")
        rng = np.random.default_rng(M + K + N + i)
        x = workloads.normal_bf16(rng, M, K, outlier_frac=0.001)
        w = workloads.nvfp4_weight(rng, N, K)
        idx = np.sort(rng.choice(N, n_mask, replace=False)).astype(np.int32) if n_mask else None
        n_out = n_mask or N
        need = nv.gemm_workspace_size(M, N, K, n_out, w4a4)
        assert 0 < need <= nv.lib().nvfp4_noalloc_scratch_bytes()
        wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
        ri = None if idx is None else helpers.dev_i32(idx)
        if w4a4:
            rc, rs = orc.quantize(x, M, K)
            a, a_s = helpers.dev_u8(rc), helpers.dev_u8(rs)
        else:
            a, a_s = helpers.dev_bf16(x), None
        want = nv.gemm(a, wc, ws, a_scales=a_s, row_idx=ri)
        g = helpers.Guarded((M, n_out), torch.bfloat16)
        _noalloc(nv, a, a_s, M, N, K, wc, ws, ri, n_out, g.t)
        g.check()
        got = helpers.host_bits(g.t)
        assert np.array_equal(got, helpers.host_bits(want))
        cols = np.sort(rng.choice(n_out, min(n_out, 128), replace=False))
        rows = idx[cols] if idx is not None else cols.astype(np.int32)
        if w4a4:
            ref = orc.gemm_w4a4(rc, rs, M, K, w.codes, w.scales, row_idx=rows.astype(np.int32))
        else:
            ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=rows.astype(np.int32))
        ok, rf, worst = helpers.gemm_close(got[:, cols], ref)
        assert ok, (rf, worst)


def test_noalloc_refuses_more_than_its_scratch(nv):
    """A call whose workspace would exceed the array returns WORKSPACE before
    any launch (W4A4 at M = 8192: its dequantized activations alone take 80 MiB)."""
    import torch
    helpers.announce("gemm_noalloc over the scratch limit")
    M, K, N = 8192, 5120, 256
    assert nv.gemm_workspace_size(M, N, K, N, True) > nv.lib().nvfp4_noalloc_scratch_bytes()
    a = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((M, K // 16), dtype=torch.uint8, device="cuda")
    wc = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    vp = ctypes.c_void_p
    rc = nv.lib().nvfp4_gemm_noalloc(nv.NVFP4, vp(a.data_ptr()), vp(s.data_ptr()), M, N, K,
                                     vp(wc.data_ptr()), vp(ws.data_ptr()), None, N, nv.BF16,
                                     vp(out.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
    assert rc == 3
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
