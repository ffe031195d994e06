"""GPU parity of the routed mixture-of-experts path: align (bit-exact),
grouped GEMM (per expert, both epilogues), combine, and the whole layer
against the oracle's token-by-token definition."""
import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("T,topk,E", [(1, 1, 1), (5, 2, 7), (32, 8, 128), (4096, 8, 128),
                                      (300, 4, 1024), (5000, 8, 100), (20000, 2, 3),
                                      (256, 8, 128), (2049, 1, 5)])
def test_align_bit_exact(nv, orc, T, topk, E):
    helpers.announce(f"moe align T={T} topk={topk} E={E}")
    if E == 128 and topk == 8:
        wl = workloads.moe(T)
        ids, gates = wl.ids, wl.gates
    else:
        rng = np.random.default_rng(T + E)
        ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
        gates = rng.random((T, topk)).astype(np.float32)
    off, gather, slot, rg = nv.moe_align(helpers.dev_i32(ids), E, helpers.dev_f32(gates))
    ro, rgat, rslot = orc.moe_align(ids, E)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(gather.cpu().numpy(), rgat)
    assert np.array_equal(slot.cpu().numpy(), rslot)
    want_rg = np.empty(T * topk, np.float32)
    want_rg[rslot.reshape(-1)] = gates.reshape(-1)
    assert np.array_equal(rg.cpu().numpy(), want_rg)


@pytest.mark.parametrize("epi,outside", [(0, False), (1, False), (0, True), (1, True)])
def test_grouped_gemm_matches_oracle(nv, orc, epi, outside):
    """Uneven groups (empty experts, one row, > 32 rows -> several chunks), with
    gather and row scale.  `outside`: some gathered rows also hold values far
    from the N(0,1) bulk (2^18, 2^-24, a bf16 subnormal)."""
    helpers.announce(f"moe grouped gemm epi={epi} outside_fp16={outside}")
    rng = np.random.default_rng(30 + epi + 2 * outside)
    E, K, N, rows = 6, 512, 96, 50
    counts = np.array([0, 1, 40, 0, 70, 9])
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, rows, K)
    if outside:
        a[3, 7] = 0x4880
        a[11, 500] = 0x3380
        a[20, 64] = 0x0005
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, rows, R).astype(np.int32)
    rs = (rng.random(R) + 0.5).astype(np.float32)
    g = helpers.Guarded((R, N // 2 if epi else N), torch.bfloat16)
    y = nv.grouped_gemm(helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
                        helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), R,
                        row_scale=helpers.dev_f32(rs), epilogue=epi, out=g.t)
    g.check()
    ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, row_scale=rs,
                           epilogue=epi)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
    assert ok, (rf, worst)


@pytest.mark.parametrize("epi,gathered,scaled", [(0, True, True), (1, True, False), (1, False, True),
                                                (0, False, False)])
def test_grouped_mfma_matches_oracle(nv, orc, epi, gathered, scaled):
    """The MFMA grouped kernel (forced for these sizes through the plan's
    grouped_mfma_min_rows): experts with 0 rows, 1 row, a partial
    256-row chunk, exactly 256 rows and several chunks; N and N/2 not multiples
    of the 256 / 128 output tile; K % 64 == 32 (a partial last K step)."""
    helpers.announce(f"moe grouped mfma epi={epi} gather={gathered} scale={scaled}")
    rng = np.random.default_rng(50 + 2 * epi + gathered + 4 * scaled)
    E, K, N = 7, 416, 352
    counts = np.array([0, 1, 300, 256, 0, 600, 37])
    R = int(counts.sum())
    rows = R if not gathered else 129
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, rows, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, rows, R).astype(np.int32) if gathered else None
    rs = (rng.random(R) + 0.5).astype(np.float32) if scaled else None
    g = helpers.Guarded((R, N // 2 if epi else N), torch.bfloat16)
    y = nv.grouped_gemm(helpers.dev_bf16(a), None if gather is None else helpers.dev_i32(gather),
                        helpers.dev_i32(off), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                        R, row_scale=None if rs is None else helpers.dev_f32(rs), epilogue=epi,
                        plan={"grouped_mfma_min_rows": 1}, out=g.t)
    g.check()
    ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, row_scale=rs,
                           epilogue=epi)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
    assert ok, (rf, worst)


# Last-chunk fills: 127, 128, 129, 255, 1 and 0 rows, with and without whole
# chunks before them; then every boundary of the 32-row activation blocks the
# tile's waves skip (a wave holds rows 64 q .. 64 q + 63 of the chunk as two
# blocks), with a partial last K step (K % 64 == 32).
_PARTIAL_CHUNKS = {
    "fills": (320, [128, 129, 255, 257, 384, 385, 127, 0, 513]),
    "blocks": (352, [1, 31, 32, 33, 64, 65, 96, 97, 160, 161, 192, 193, 224, 225, 287]),
}


@pytest.mark.parametrize("case", sorted(_PARTIAL_CHUNKS))
@pytest.mark.parametrize("epi", [0, 1])
def test_grouped_mfma_partial_chunks(nv, orc, epi, case):
    """Experts with partly filled 256-row chunks through the grouped MFMA
    kernel: every row against the oracle, guarded output."""
    helpers.announce(f"moe grouped mfma partial chunks {case} epi={epi}")
    rng = np.random.default_rng(80 + epi + (10 if case == "blocks" else 0))
    K, counts = _PARTIAL_CHUNKS[case]
    counts = np.array(counts)
    E, N = len(counts), 288
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, 700, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, 700, R).astype(np.int32)
    rs = (rng.random(R) + 0.5).astype(np.float32)
    g = helpers.Guarded((R, N // 2 if epi else N), torch.bfloat16)
    y = nv.grouped_gemm(helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
                        helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), R,
                        row_scale=helpers.dev_f32(rs), epilogue=epi,
                        plan={"grouped_mfma_min_rows": 1}, out=g.t)
    g.check()
    ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, row_scale=rs,
                           epilogue=epi)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
    assert ok, (rf, worst)


def test_combine_matches_oracle(nv, orc):
    helpers.announce("moe combine")
    rng = np.random.default_rng(40)
    T, topk, H = 33, 8, 2048
    y = workloads.normal_bf16(rng, T * topk, H)
    slot = rng.permutation(T * topk).astype(np.int32).reshape(T, topk)
    g = helpers.Guarded((T, H), torch.bfloat16)
    got = helpers.host_bits(nv.moe_combine(helpers.dev_bf16(y), helpers.dev_i32(slot), out=g.t))
    g.check()
    ref = orc.moe_combine(y, slot, T, topk, H)
    ok, rf, worst = helpers.gemm_close(got, ref)
    assert ok, (rf, worst)


def _dev_g(g):
    return None if g is None else helpers.dev_f32(g)


def _layer(nv, wl, g1=None, g2=None):
    import torch
    out = nv.moe_layer(helpers.dev_bf16(wl.x), helpers.dev_i32(wl.ids), helpers.dev_f32(wl.gates),
                       helpers.dev_u8(wl.w1.codes), helpers.dev_u8(wl.w1.scales),
                       helpers.dev_u8(wl.w2.codes), helpers.dev_u8(wl.w2.scales),
                       w1_global=_dev_g(g1), w2_global=_dev_g(g2))
    torch.cuda.synchronize()
    return helpers.host_bits(out)


def _slot_magnitude(orc, wl, toks, g1=None, g2=None):
    """sum_j |y_j| per output element, from the oracle's own grouped steps: the
    scale of the terms the combine adds (each stored in bf16).  g1 / g2: the
    experts' global scales of two-level weights."""
    ids, gates = wl.ids[toks], wl.gates[toks]
    T, topk = ids.shape
    E = wl.w1.codes.shape[0]
    I = wl.w2.codes.shape[2] * 2
    H = wl.x.shape[1]
    off, gather, slot = orc.moe_align(ids, E)
    R = T * topk
    act = orc.bf16_round(orc.grouped_gemm(wl.x[toks], H, gather, off, E, R, 2 * I, wl.w1.codes,
                                          wl.w1.scales, epilogue=1, w_global=g1))
    rg = np.empty(R, np.float32)
    rg[slot.reshape(-1)] = gates.reshape(-1)
    y = helpers.bf16_bits_to_f64(orc.bf16_round(orc.grouped_gemm(
        act, I, None, off, E, R, H, wl.w2.codes, wl.w2.scales, row_scale=rg, w_global=g2)))
    return np.abs(y)[slot].sum(axis=1)


def _layer_close(got_bits, ref, mag):
    """Layer tolerance: relative Frobenius <= 1e-3 (as for a GEMM output) and
    every element within 1e-2*(sum_j |y_j| + 1): the output is a sum of topk
    terms that are each stored in bf16, so its element error scales with the
    terms, not with their (possibly cancelling) sum."""
    g = helpers.bf16_bits_to_f64(got_bits)
    import oracle
    r = helpers.bf16_bits_to_f64(oracle.bf16_round(ref))
    rf = np.linalg.norm(g - r) / np.linalg.norm(r)
    worst = np.max(np.abs(g - r) / (1e-2 * (mag + 1.0)))
    return rf <= 1e-3 and worst <= 1.0, rf, worst


def test_moe_layer_decode_full(nv, orc):
    """T = 32 decode batch, 128 experts, top-8, H = 2048, I = 768: every token."""
    helpers.announce("moe layer T=32 full")
    wl = workloads.moe(32)
    got = _layer(nv, wl)
    ref = orc.moe_layer(wl.x, wl.ids, wl.gates, 128, 768, wl.w1.codes, wl.w1.scales,
                        wl.w2.codes, wl.w2.scales)
    ok, rf, worst = _layer_close(got, ref, _slot_magnitude(orc, wl, np.arange(32)))
    assert ok, (rf, worst)


def test_moe_layer_steps_chained(nv, orc):
    """Every GPU step of the T = 32 layer against the oracle fed the GPU's own
    inputs to that step: each stored intermediate is a plain GEMM output and
    meets the GEMM tolerance elementwise."""
    import torch
    helpers.announce("moe layer T=32 chained steps")
    wl = workloads.moe(32)
    E, H, I = 128, 2048, 768
    T, topk = wl.ids.shape
    R = T * topk
    w1c, w1s = helpers.dev_u8(wl.w1.codes), helpers.dev_u8(wl.w1.scales)
    w2c, w2s = helpers.dev_u8(wl.w2.codes), helpers.dev_u8(wl.w2.scales)
    off, gather, slot, rg = nv.moe_align(helpers.dev_i32(wl.ids), E, helpers.dev_f32(wl.gates))
    act = nv.grouped_gemm(helpers.dev_bf16(wl.x), gather, off, w1c, w1s, R, epilogue=1)
    y = nv.grouped_gemm(act, None, off, w2c, w2s, R, row_scale=rg)
    out = nv.moe_combine(y, slot)
    torch.cuda.synchronize()
    off_h, gather_h, slot_h = off.cpu().numpy(), gather.cpu().numpy(), slot.cpu().numpy()
    rg_h, act_h, y_h = rg.cpu().numpy(), helpers.host_bits(act), helpers.host_bits(y)
    ref_act = orc.grouped_gemm(wl.x, H, gather_h, off_h, E, R, 2 * I, wl.w1.codes, wl.w1.scales,
                               epilogue=1)
    assert helpers.gemm_close(act_h, ref_act)[0]
    ref_y = orc.grouped_gemm(act_h, I, None, off_h, E, R, H, wl.w2.codes, wl.w2.scales,
                             row_scale=rg_h)
    ok, rf, worst = helpers.gemm_close(y_h, ref_y)
    assert ok, (rf, worst)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(out), orc.moe_combine(y_h, slot_h, T, topk, H))
    assert ok, (rf, worst)


def test_moe_layer_prefill_sampled(nv, orc):
    """T = 4096 prefill batch: the full layer on the GPU, 48 sampled tokens
    recomputed by the oracle."""
    helpers.announce("moe layer T=4096 sampled")
    wl = workloads.moe(4096)
    got = _layer(nv, wl)
    toks = np.sort(np.random.default_rng(41).choice(4096, 48, replace=False))
    ref = orc.moe_layer(wl.x[toks], wl.ids[toks], wl.gates[toks], 128, 768, wl.w1.codes,
                        wl.w1.scales, wl.w2.codes, wl.w2.scales)
    ok, rf, worst = _layer_close(got[toks], ref, _slot_magnitude(orc, wl, toks))
    assert ok, (rf, worst)


def _sub_problem(rows, off_h, E):
    """Offsets of a grouped problem holding only the grouped rows `rows`
    (sorted), each still with its expert: the expert of row r is the e with
    off[e] <= r < off[e+1]."""
    ex = np.searchsorted(off_h, rows, side="right") - 1
    counts = np.bincount(ex, minlength=E)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _chained(nv, orc, wl, n_rows=None, n_tok=None, seed=0, down_fp32_bound=False, g1=None,
             g2=None):
    """Every GPU step of the layer against the oracle fed the GPU's own inputs
    to that step, at the GEMM tolerance element by element: align bit-exact,
    then the gate/up grouped GEMM with SwiGLU, the down grouped GEMM with the
    gate weights and the combine, each on all rows (n_rows None) or on a
    seeded sample of grouped rows / tokens (the oracle recomputes a grouped
    problem of just those rows, each with its own expert).  down_fp32_bound:
    the down projection's element bound also admits the fp32 summation error
    bound I * 2^-24 * sum_k |a_k w_k g_r| of each output.  g1 / g2: the
    experts' global scales of two-level weights (fp32 [E])."""
    E = wl.w1.codes.shape[0]
    H = wl.x.shape[1]
    I = wl.w2.codes.shape[2] * 2
    T, topk = wl.ids.shape
    R = T * topk
    w1c, w1s = helpers.dev_u8(wl.w1.codes), helpers.dev_u8(wl.w1.scales)
    w2c, w2s = helpers.dev_u8(wl.w2.codes), helpers.dev_u8(wl.w2.scales)
    off, gather, slot, rg = nv.moe_align(helpers.dev_i32(wl.ids), E, helpers.dev_f32(wl.gates))
    act = nv.grouped_gemm(helpers.dev_bf16(wl.x), gather, off, w1c, w1s, R, epilogue=1,
                          w_global=_dev_g(g1))
    y = nv.grouped_gemm(act, None, off, w2c, w2s, R, row_scale=rg, w_global=_dev_g(g2))
    out = nv.moe_combine(y, slot)
    torch.cuda.synchronize()
    off_h, gather_h, slot_h = off.cpu().numpy(), gather.cpu().numpy(), slot.cpu().numpy()
    rg_h, act_h, y_h = rg.cpu().numpy(), helpers.host_bits(act), helpers.host_bits(y)
    ro, rgat, rslot = orc.moe_align(wl.ids, E)
    assert np.array_equal(off_h, ro) and np.array_equal(gather_h, rgat)
    assert np.array_equal(slot_h, rslot)
    rng = np.random.default_rng(seed)
    rows = np.arange(R) if n_rows is None else np.sort(rng.choice(R, n_rows, replace=False))
    toks = np.arange(T) if n_tok is None else np.sort(rng.choice(T, n_tok, replace=False))
    so = _sub_problem(rows, off_h, E)
    ref_act = orc.grouped_gemm(wl.x, H, gather_h[rows], so, E, len(rows), 2 * I, wl.w1.codes,
                               wl.w1.scales, epilogue=1, w_global=g1)
    ok, rf, worst = helpers.gemm_close(act_h[rows], ref_act)
    assert ok, ("gate/up", rf, worst)
    ref_y = orc.grouped_gemm(np.ascontiguousarray(act_h[rows]), I, None, so, E, len(rows), H,
                             wl.w2.codes, wl.w2.scales, row_scale=rg_h[rows], w_global=g2)
    extra = None
    if down_fp32_bound:
        a_abs = np.ascontiguousarray(act_h[rows] & 0x7FFF)
        mag = orc.grouped_gemm(a_abs, I, None, so, E, len(rows), H, wl.w2.codes & 0x77,
                               wl.w2.scales, row_scale=np.abs(rg_h[rows]), w_global=g2)
        extra = I * 2.0 ** -24 * mag
        ok_bj, _, worst_bj = helpers.gemm_close(y_h[rows], ref_y)
        print(f"[down] BJ element bound alone: ok={ok_bj} worst ratio {worst_bj:.2f}", flush=True)
    ok, rf, worst = helpers.gemm_close(y_h[rows], ref_y, abs_extra=extra)
    assert ok, ("down", rf, worst)
    ref_out = orc.moe_combine(y_h, np.ascontiguousarray(slot_h[toks]), len(toks), topk, H)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(out)[toks], ref_out)
    assert ok, ("combine", rf, worst)


def test_moe_layer_prefill_steps_chained_sampled(nv, orc):
    """T = 4096 at full size (the MFMA grouped kernel): every step held to the
    GEMM tolerance element by element on 96 sampled grouped rows (experts of
    every popularity) and 64 sampled tokens, the oracle fed the GPU's own
    inputs to each step."""
    helpers.announce("moe layer T=4096 chained steps, sampled rows")
    _chained(nv, orc, workloads.moe(4096), n_rows=96, n_tok=64, seed=43)


def test_moe_layer_steps_chained_dense_scales(nv, orc):
    """T = 32 with the dense layers' scale distribution (exponent fields 3..9,
    2^-4 .. 2^2 before the mantissa) instead of the checkpoint-like expert
    scales: the SwiGLU outputs grow to ~10^5 and the down projection's 768-term
    sums cancel far below their terms, so its element bound 1e-2*(|ref|+1)
    cannot hold for fp32 accumulation; that step is held to it plus the fp32
    summation error bound of each output (relative Frobenius <= 1e-3 as
    always).  Align, gate/up and combine meet the plain GEMM tolerance."""
    helpers.announce("moe layer T=32 chained steps, dense-layer scales")
    _chained(nv, orc, workloads.moe(32, exp_field=(3, 9)), down_fp32_bound=True)


def test_grouped_long_k_few_rows(nv, orc):
    """A K past the grouped GEMV's LDS staging (5,120 > 4,864) with decode-like
    row counts runs the MFMA kernel; every row against the oracle, both
    epilogues, guarded outputs."""
    rng = np.random.default_rng(60)
    E, K, N = 5, 5120, 96
    counts = np.array([1, 3, 0, 5, 2])
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, 7, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, 7, R).astype(np.int32)
    for epi in (0, 1):
        helpers.announce(f"moe grouped long K={K} epi={epi}")
        g = helpers.Guarded((R, N // 2 if epi else N), torch.bfloat16)
        y = nv.grouped_gemm(helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
                            helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), R, epilogue=epi,
                            out=g.t)
        g.check()
        ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, epilogue=epi)
        ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
        assert ok, (epi, rf, worst)


# ---- two-level expert weights (one fp32 global scale per expert) ---------------

@pytest.mark.parametrize("kernel,epi", [("gemv", 0), ("gemv", 1), ("mfma", 0), ("mfma", 1)])
def test_grouped_two_level_matches_oracle(nv, orc, kernel, epi):
    """nvfp4_grouped_gemm_scaled on both grouped kernels: block scales near the
    top of E4M3 (up to 448) and per-expert global scales 2^-14 .. 2^-12 (one
    expert's exactly 1); uneven experts (empty, one row, several chunks), with
    gather and row scale, guarded output.  Unit global scales reproduce
    nvfp4_grouped_gemm bit for bit."""
    helpers.announce(f"moe grouped two-level kernel={kernel} epi={epi}")
    rng = np.random.default_rng(70 + epi + 2 * (kernel == "mfma"))
    if kernel == "gemv":
        E, K, N, rows = 6, 512, 96, 50
        counts = np.array([0, 1, 40, 0, 70, 9])
        plan = {"grouped_mfma_min_rows": 1 << 20}
    else:
        E, K, N, rows = 5, 416, 352, 129
        counts = np.array([1, 300, 0, 256, 37])
        plan = {"grouped_mfma_min_rows": 1}
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, rows, K)
    w = workloads.nvfp4_weight(rng, E, N, K, exp_field=workloads.MOE_TWO_LEVEL_EXP_FIELD)
    wg = workloads.expert_global_scales(rng, E)
    wg[2] = 1.0
    gather = rng.integers(0, rows, R).astype(np.int32)
    rs = (rng.random(R) + 0.5).astype(np.float32)
    width = N // 2 if epi else N
    args = (helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
            helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), R)
    g = helpers.Guarded((R, width), torch.bfloat16)
    y = nv.grouped_gemm(*args, row_scale=helpers.dev_f32(rs), epilogue=epi, plan=plan,
                        w_global=helpers.dev_f32(wg), out=g.t)
    g.check()
    ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, row_scale=rs,
                           epilogue=epi, w_global=wg)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
    assert ok, (rf, worst)
    ones = nv.grouped_gemm(*args, row_scale=helpers.dev_f32(rs), epilogue=epi, plan=plan,
                           w_global=helpers.dev_f32(np.ones(E, np.float32)))
    plain = nv.grouped_gemm(*args, row_scale=helpers.dev_f32(rs), epilogue=epi, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(ones, plain)


def test_moe_layer_two_level_decode_full(nv, orc):
    """T = 32 decode batch with two-level expert weights through the binding's
    layer (both global-scale arrays): every token against the oracle's
    token-by-token layer."""
    helpers.announce("moe layer two-level T=32 full")
    wl, g1, g2 = workloads.moe_two_level(32)
    got = _layer(nv, wl, g1, g2)
    ref = orc.moe_layer(wl.x, wl.ids, wl.gates, 128, 768, wl.w1.codes, wl.w1.scales,
                        wl.w2.codes, wl.w2.scales, w1_global=g1, w2_global=g2)
    ok, rf, worst = _layer_close(got, ref, _slot_magnitude(orc, wl, np.arange(32), g1, g2))
    assert ok, (rf, worst)


def test_moe_layer_two_level_steps_chained(nv, orc):
    """Every step of the two-level layer at T = 32 (grouped GEMV) on all rows and
    at T = 4096 (MFMA grouped kernel) on sampled rows and tokens, the oracle fed
    the GPU's own inputs to each step."""
    helpers.announce("moe layer two-level T=32 chained steps")
    wl, g1, g2 = workloads.moe_two_level(32, seed=5)
    _chained(nv, orc, wl, g1=g1, g2=g2)
    helpers.announce("moe layer two-level T=4096 chained steps, sampled rows")
    wl, g1, g2 = workloads.moe_two_level(4096, seed=6)
    _chained(nv, orc, wl, n_rows=96, n_tok=64, seed=44, g1=g1, g2=g2)
