"""GPU parity of the draft proposal (nvfp4_topk, nvfp4_head_topk) against the
oracle.

Selection on given fp32 logits is bit-exact (values and ids).  For the fused
head, one-hot activations make every logit a single exact product, so ids and
values are compared bit for bit; with random activations the kernel's fp32
logits differ from the exact ones by rounding, so the proposal is checked for
validity: distinct kept ids, values within the fp32 summation bound
K * 2^-24 * sum|x||w| of their exact logits, non-increasing, and no id below
the exact k-th best by more than twice that bound."""
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


def _logits(kind, M, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((M, n)).astype(np.float32)
    if kind == "ties":  # few distinct values, both zeros, infinities
        pool = np.array([-np.inf, -2.0, -0.5, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf], np.float32)
        return pool[rng.integers(0, len(pool), size=(M, n))]
    if kind == "zeros":  # every logit +-0: the order is the sign, then the column
        v = np.zeros((M, n), np.float32)
        v[rng.random((M, n)) < 0.5] = -0.0
        return v
    raise ValueError(kind)


def _check_exact(nv, orc, v, k, ids_map=None):
    import torch
    ld = torch.from_numpy(v).cuda()
    im = None if ids_map is None else helpers.dev_i32(ids_map)
    gval = helpers.Guarded((v.shape[0], k), torch.float32)
    gids = helpers.Guarded((v.shape[0], k), torch.int32)
    gv, gi = nv.topk(ld, k, ids_map=im, values=gval.t, ids=gids.t)
    gval.check()
    gids.check()
    gv, gi = gv.cpu().numpy(), gi.cpu().numpy()
    ov, oi = orc.topk(v, k, ids_map=ids_map)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("kind,M,n,k", [
    ("normal", 1, 7, 7),            # k = n, a single short chunk
    ("ties", 3, 2048, 64),          # exactly one chunk
    ("ties", 2, 2049, 256),         # two chunks, the second holds one element
    ("normal", 4, 32768, 8),        # the masked head width
    ("ties", 5, 32768, 1),          # argmax with many ties
    ("zeros", 2, 5000, 100),
    ("normal", 1, 248320, 64),      # the full vocabulary: three levels
    ("ties", 33, 4099, 3),          # more rows than one decode chunk; ragged last chunk
])
def test_topk_matches_oracle(nv, orc, kind, M, n, k):
    helpers.announce(f"topk {kind} M={M} n={n} k={k}")
    _check_exact(nv, orc, _logits(kind, M, n, seed=M * 7 + n + k), k)


def test_topk_ids_map(nv, orc):
    helpers.announce("topk ids_map M=3 n=6000 k=16")
    rng = np.random.default_rng(41)
    idx = np.sort(rng.choice(100000, 6000, replace=False)).astype(np.int32)
    _check_exact(nv, orc, _logits("ties", 3, 6000, 42), 16, ids_map=idx)


def test_topk_rejects_k_above_n(nv):
    import torch
    ld = torch.zeros((2, 10), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="INVALID"):
        nv.topk(ld, 11)
    with pytest.raises(RuntimeError, match="NOT_SUPPORTED"):
        nv.topk(torch.zeros((1, 1000), dtype=torch.float32, device="cuda"), 257)


@pytest.mark.parametrize("M", [1, 8, 32, 70])
def test_head_topk_one_hot_exact(nv, orc, M):
    """x rows are unit vectors, so each logit is one weight value (exact in
    fp32 whatever the summation order): the proposal must match the oracle bit
    for bit, ties included.  M = 70 takes the MFMA GEMM path."""
    helpers.announce(f"head_topk one-hot M={M}")
    rng = np.random.default_rng(50 + M)
    N, K, n_keep, k = 40000, 256, 32768, 8
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, n_keep, replace=False)).astype(np.int32)
    x = np.zeros((M, K))
    x[np.arange(M), rng.integers(0, K, size=M)] = rng.choice([1.0, -2.0, 0.5], size=M)
    xb = helpers.f64_to_bf16_bits_exact(x)
    import torch
    gval = helpers.Guarded((M, k), torch.float32)
    gids = helpers.Guarded((M, k), torch.int32)
    gv, gi = nv.head_topk(helpers.dev_bf16(xb), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                          k, row_idx=helpers.dev_i32(idx), values=gval.t, ids=gids.t)
    gval.check()
    gids.check()
    ov, oi, _ = orc.head_topk(xb, M, K, w.codes, w.scales, k, row_idx=idx)
    assert np.array_equal(gi.cpu().numpy(), oi)
    assert np.array_equal(gv.cpu().numpy().view(np.uint32), ov.astype(np.float32).view(np.uint32))


def _abs_bound(orc, x, M, K, w, idx):
    """K * 2^-24 * sum_k |x||w| per logit: the fp32 summation error bound."""
    xa = (np.asarray(x, np.uint16) & 0x7FFF).astype(np.uint16)
    ca = (np.asarray(w.codes) & 0x77).astype(np.uint8)
    s = orc.gemm_w4a16(xa, M, K, ca, w.scales, row_idx=idx)
    return K * 2.0 ** -24 * s.max(axis=1, keepdims=True) + 1e-30


def test_head_topk_full_size_valid(nv, orc):
    """The masked head at full size (32,768 of 248,320 rows, K = 5120) for M in
    {1, 8, 32}, k = 8, in the configuration the benchmark times."""
    K, N = workloads.HIDDEN, workloads.VOCAB
    w = workloads.decode_weights(K, N)
    idx = workloads.decode_masked_rows()
    wc, ws, ri = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), helpers.dev_i32(idx)
    k = 8
    for M in workloads.DECODE_M:
        helpers.announce(f"head_topk full size M={M} k={k}")
        x = workloads.decode_activations(M, K)
        gv, gi = nv.head_topk(helpers.dev_bf16(x), wc, ws, k, row_idx=ri)
        _, _, logits = orc.head_topk(x, M, K, w.codes, w.scales, k, row_idx=idx)
        tol = _abs_bound(orc, x, M, K, w, idx)
        for m in range(M):
            assert helpers.topk_valid(gv.cpu().numpy()[m:m + 1], gi.cpu().numpy()[m:m + 1],
                                      logits[m:m + 1], idx, float(tol[m, 0])), f"M={M} row {m}"


def test_head_topk_equals_gemm_then_topk(nv):
    """The fused entry point returns what nvfp4_gemm (fp32 out) followed by
    nvfp4_topk returns, bit for bit (same kernels, same sums)."""
    import torch
    helpers.announce("head_topk vs gemm+topk M=8")
    rng = np.random.default_rng(60)
    N, K, n_keep, k = 9000, 512, 4000, 32
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, n_keep, replace=False)).astype(np.int32)
    x = workloads.normal_bf16(rng, 8, K)
    xd, wc, ws, ri = helpers.dev_bf16(x), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), \
        helpers.dev_i32(idx)
    gv, gi = nv.head_topk(xd, wc, ws, k, row_idx=ri)
    logits = nv.gemm(xd, wc, ws, row_idx=ri, out_dtype=torch.float32)
    tv, ti = nv.topk(logits, k, ids_map=ri)
    assert torch.equal(gi, ti)
    assert torch.equal(gv.view(torch.int32), tv.view(torch.int32))
