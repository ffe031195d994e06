"""Pins of the oracle's routed mixture-of-experts functions: routing preparation
against Python's stable sort, the grouped GEMM per expert against numpy BLAS on
independently dequantized weights, the combine against numpy sums, and the
whole layer against (a) a dense two-layer MLP when there is one expert and one
slot and (b) the composition align -> grouped GEMM -> grouped GEMM -> combine."""
import numpy as np
import pytest

import helpers
import workloads


def _silu(z):
    return z / (1.0 + np.exp(-z))


def test_moe_align_matches_stable_sort(orc):
    rng = np.random.default_rng(20)
    for T, topk, E in [(1, 1, 1), (7, 2, 5), (64, 8, 128), (300, 8, 16)]:
        ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
        off, gather, slot = orc.moe_align(ids, E)
        flat = ids.reshape(-1)
        order = sorted(range(T * topk), key=lambda p: (flat[p], p))  # stable by expert
        assert list(gather) == [p // topk for p in order]
        counts = np.bincount(flat, minlength=E)
        assert list(off) == [0] + list(np.cumsum(counts))
        for r, p in enumerate(order):
            assert slot.reshape(-1)[p] == r


def test_moe_align_rejects_bad_id(orc):
    with pytest.raises(ValueError):
        orc.moe_align(np.array([[0, 5]], np.int32), 4)


def test_grouped_gemm_matches_blas_per_expert(orc):
    rng = np.random.default_rng(21)
    E, K, N, rows = 4, 256, 48, 30
    a = workloads.normal_bf16(rng, rows, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, rows, size=50).astype(np.int32)
    cuts = np.sort(rng.integers(0, 51, size=E - 1))
    off = np.concatenate([[0], cuts, [50]]).astype(np.int32)
    rs = rng.random(50).astype(np.float32)
    A = helpers.bf16_bits_to_f64(a)
    for epi in (0, 1):
        for use_scale in (False, True):
            got = orc.grouped_gemm(a, K, gather, off, E, 50, N, w.codes, w.scales,
                                   row_scale=rs if use_scale else None, epilogue=epi)
            for e in range(E):
                We = helpers.dequant_independent(w.codes[e], w.scales[e])
                h = A[gather[off[e]:off[e + 1]]] @ We.T
                ref = _silu(h[:, :N // 2]) * h[:, N // 2:] if epi == 1 else h
                if use_scale:
                    ref = ref * rs[off[e]:off[e + 1], None].astype(np.float64)
                assert np.allclose(got[off[e]:off[e + 1]], ref, rtol=1e-12, atol=1e-9)


def test_grouped_gemm_without_gather_reads_row_r(orc):
    rng = np.random.default_rng(22)
    E, K, N, R = 3, 128, 16, 12
    a = workloads.normal_bf16(rng, R, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    off = np.array([0, 5, 5, 12], np.int32)
    got = orc.grouped_gemm(a, K, None, off, E, R, N, w.codes, w.scales)
    ident = orc.grouped_gemm(a, K, np.arange(R, dtype=np.int32), off, E, R, N, w.codes, w.scales)
    assert np.array_equal(got, ident)


def test_combine_matches_numpy(orc):
    rng = np.random.default_rng(23)
    T, topk, H = 10, 3, 64
    y = workloads.normal_bf16(rng, T * topk, H)
    slot = rng.permutation(T * topk).astype(np.int32).reshape(T, topk)
    got = orc.moe_combine(y, slot, T, topk, H)
    Y = helpers.bf16_bits_to_f64(y)
    ref = Y[slot].sum(axis=1)
    assert np.allclose(got, ref, rtol=1e-15, atol=0)


def test_moe_layer_one_expert_is_dense_mlp(orc):
    """E = 1, topk = 1, gate 1.0: the layer is bf16(silu(x W_g^T) * (x W_u^T)) W_d^T
    with the same bf16 storage points, computed here with numpy BLAS."""
    rng = np.random.default_rng(24)
    T, H, I = 6, 256, 64
    x = workloads.normal_bf16(rng, T, H)
    w1 = workloads.nvfp4_weight(rng, 1, 2 * I, H)
    w2 = workloads.nvfp4_weight(rng, 1, H, I)
    ids = np.zeros((T, 1), np.int32)
    gates = np.ones((T, 1), np.float32)
    got = orc.moe_layer(x, ids, gates, 1, I, w1.codes, w1.scales, w2.codes, w2.scales)
    X = helpers.bf16_bits_to_f64(x)
    W1 = helpers.dequant_independent(w1.codes[0], w1.scales[0])
    W2 = helpers.dequant_independent(w2.codes[0], w2.scales[0])
    h = X @ W1.T
    act = helpers.bf16_bits_to_f64(orc.bf16_round(_silu(h[:, :I]) * h[:, I:]))
    y = helpers.bf16_bits_to_f64(orc.bf16_round(act @ W2.T))
    # the single-slot sum is the stored bf16 y itself
    assert np.array_equal(got, y) or np.allclose(got, y, rtol=0, atol=0)


def test_moe_layer_equals_grouped_composition(orc):
    """The token-by-token layer equals align -> grouped GEMM (SwiGLU, bf16) ->
    grouped GEMM (gate weights, bf16) -> combine, for a Zipf-routed batch."""
    E, topk, H, I, T = 8, 2, 128, 32, 24
    wl = workloads.moe(T, E=E, topk=topk, H=H, I=I, seed=3)
    layer = orc.moe_layer(wl.x, wl.ids, wl.gates, E, I, wl.w1.codes, wl.w1.scales,
                          wl.w2.codes, wl.w2.scales)
    off, gather, slot = orc.moe_align(wl.ids, E)
    R = T * topk
    act = orc.bf16_round(orc.grouped_gemm(wl.x, H, gather, off, E, R, 2 * I, wl.w1.codes,
                                          wl.w1.scales, epilogue=1))
    # gate weight of row r: the assignment p that landed in r
    p_of_r = np.empty(R, np.int64)
    p_of_r[slot.reshape(-1)] = np.arange(R)
    g = wl.gates.reshape(-1)[p_of_r].astype(np.float32)
    y = orc.bf16_round(orc.grouped_gemm(act, I, None, off, E, R, H, wl.w2.codes, wl.w2.scales,
                                        row_scale=g))
    comb = orc.moe_combine(y, slot, T, topk, H)
    assert np.allclose(layer, comb, rtol=1e-12, atol=1e-12)


def test_zipf_routing_properties():
    wl = workloads.moe(512)
    ids, gates = wl.ids, wl.gates
    assert ids.shape == (512, 8) and gates.shape == (512, 8)
    assert all(len(set(r)) == 8 for r in ids)             # distinct experts per token
    assert np.allclose(gates.sum(axis=1), 1.0, atol=1e-6)  # softmax-normalised
    assert np.all(np.diff(gates, axis=1) <= 1e-7)          # kept in descending score order
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.max() > 10 * max(1, np.median(counts)) or counts.max() > 3 * np.median(counts)


# ---- two-level expert weights (one fp32 global scale per expert) ----------------

def _two_level_experts(orc, seed, E, N, K):
    """bf16 weights of E experts, each of its own magnitude, quantized expert by
    expert with the oracle's offline quantizer; expert 1 is all zero."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((E, N, K)).astype(np.float32)
    w *= (np.float32(2.0) ** rng.integers(-9, 3, size=(E, 1, 1))).astype(np.float32)
    w *= (1.0 + rng.random((E, 1, 1))).astype(np.float32)  # not a power of two
    w[1] = 0.0
    bits = workloads.f32_to_bf16_bits(w)
    codes = np.empty((E, N, K // 2), np.uint8)
    scales = np.empty((E, N, K // 16), np.uint8)
    g = np.empty(E, np.float32)
    for e in range(E):
        codes[e], scales[e], g[e] = orc.quantize_weight(bits[e], N, K)
    return bits, codes, scales, g


def test_expert_global_scales_are_binary32_divisions(orc):
    bits, _, scales, g = _two_level_experts(orc, 25, 5, 32, 128)
    for e in range(5):
        amax = np.abs(helpers.bf16_bits_to_f64(bits[e])).max()
        want = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(2688.0)
        assert g[e] == want, e
        if amax > 0:  # the expert's largest block gets the largest finite scale
            assert scales[e].max() == 0x7E


def test_grouped_two_level_matches_blas_per_expert(orc):
    """Expert e's output is g_e times the BLAS product of its dequantized
    weights, before SwiGLU and the row scale."""
    rng = np.random.default_rng(26)
    E, K, N, rows, R = 4, 256, 64, 30, 50
    _, codes, scales, g = _two_level_experts(orc, 27, E, N, K)
    a = workloads.normal_bf16(rng, rows, K)
    gather = rng.integers(0, rows, size=R).astype(np.int32)
    off = np.concatenate([[0], np.sort(rng.integers(0, R + 1, size=E - 1)), [R]]).astype(np.int32)
    rs = rng.random(R).astype(np.float32)
    A = helpers.bf16_bits_to_f64(a)
    for epi in (0, 1):
        for use_scale in (False, True):
            got = orc.grouped_gemm(a, K, gather, off, E, R, N, codes, scales,
                                   row_scale=rs if use_scale else None, epilogue=epi, w_global=g)
            for e in range(E):
                We = helpers.dequant_independent(codes[e], scales[e])
                h = (A[gather[off[e]:off[e + 1]]] @ We.T) * float(g[e])
                ref = _silu(h[:, :N // 2]) * h[:, N // 2:] if epi == 1 else h
                if use_scale:
                    ref = ref * rs[off[e]:off[e + 1], None].astype(np.float64)
                assert np.allclose(got[off[e]:off[e + 1]], ref, rtol=1e-12, atol=1e-12)


def test_grouped_two_level_unit_and_power_of_two_scales(orc):
    """Unit global scales are the single-level product; power-of-two ones scale
    the plain product exactly and are not confused between experts."""
    rng = np.random.default_rng(28)
    E, K, N, R = 3, 128, 32, 20
    a = workloads.normal_bf16(rng, R, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    off = np.array([0, 7, 7, 20], np.int32)
    plain = orc.grouped_gemm(a, K, None, off, E, R, N, w.codes, w.scales)
    ones = orc.grouped_gemm(a, K, None, off, E, R, N, w.codes, w.scales,
                            w_global=np.ones(E, np.float32))
    assert np.array_equal(plain, ones)
    j = np.array([-3, 7, 2])
    g = np.ldexp(np.ones(E), j).astype(np.float32)
    got = orc.grouped_gemm(a, K, None, off, E, R, N, w.codes, w.scales, w_global=g)
    for e in range(E):
        sl = slice(off[e], off[e + 1])
        assert np.array_equal(got[sl], plain[sl] * 2.0 ** j[e])


def test_moe_layer_two_level_equals_grouped_composition(orc):
    E, topk, H, I, T = 8, 2, 128, 32, 24
    wl, g1, g2 = workloads.moe_two_level(T, E=E, topk=topk, H=H, I=I, seed=4)
    layer = orc.moe_layer(wl.x, wl.ids, wl.gates, E, I, wl.w1.codes, wl.w1.scales,
                          wl.w2.codes, wl.w2.scales, w1_global=g1, w2_global=g2)
    off, gather, slot = orc.moe_align(wl.ids, E)
    R = T * topk
    act = orc.bf16_round(orc.grouped_gemm(wl.x, H, gather, off, E, R, 2 * I, wl.w1.codes,
                                          wl.w1.scales, epilogue=1, w_global=g1))
    p_of_r = np.empty(R, np.int64)
    p_of_r[slot.reshape(-1)] = np.arange(R)
    gate = wl.gates.reshape(-1)[p_of_r].astype(np.float32)
    y = orc.bf16_round(orc.grouped_gemm(act, I, None, off, E, R, H, wl.w2.codes, wl.w2.scales,
                                        row_scale=gate, w_global=g2))
    comb = orc.moe_combine(y, slot, T, topk, H)
    assert np.allclose(layer, comb, rtol=1e-12, atol=1e-12)
    # the two-level layer is not the single-level one (the scales are used)
    plain = orc.moe_layer(wl.x, wl.ids, wl.gates, E, I, wl.w1.codes, wl.w1.scales,
                          wl.w2.codes, wl.w2.scales)
    assert not np.allclose(layer, plain)
    # activations stay of order one to ten, like the single-level workload's
    assert 0.05 < np.sqrt(np.mean(layer ** 2)) < 50


def test_two_level_workload_scales():
    wl, g1, g2 = workloads.moe_two_level(16, E=6, H=128, I=32, seed=1)
    for w in (wl.w1, wl.w2):
        assert w.scales.max() <= 0x7E and (w.scales >> 3).min() >= 11
    for g in (g1, g2):
        assert g.dtype == np.float32 and g.shape == (6,)
        assert np.all((g >= 2.0 ** -14) & (g < 2.0 ** -12))
