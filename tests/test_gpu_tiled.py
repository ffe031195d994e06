"""GPU parity of the tiled weight layout: nvfp4_tile_weight byte-identical to the
oracle's tile_weight, and nvfp4_gemm_tiled against the fp64 oracle's product on
the row-major weights (relative Frobenius error <= 1e-3, every element within
1e-2*(|ref|+1); bf16 outputs against the oracle rounded once to bf16), with
guard-padded outputs, every built launch layout, ragged shapes, full-size
sampled decode shapes, and bit-identity with the row-major kernel of the same
launch layout."""
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


def _tiled(nv, w):
    return nv.tile_weight(helpers.dev_u8(w.codes), helpers.dev_u8(w.scales))


def _run(nv, x, wt, N, out_f32=False, plan=None):
    import torch
    dt = torch.float32 if out_f32 else torch.bfloat16
    g = helpers.Guarded((x.shape[0], N), dt)
    y = nv.gemm_tiled(helpers.dev_bf16(x), wt, N, out_dtype=dt, plan=plan, out=g.t)
    g.check()
    return y.cpu().numpy() if out_f32 else helpers.host_bits(y)


def _assert_close(got, ref, out_f32=False, what=""):
    ok, rf, worst = helpers.gemm_close(got, ref, out_is_bf16=not out_f32)
    assert ok, f"{what}: rel_frob={rf:.3e} worst_elem_ratio={worst:.3f}"


@pytest.mark.parametrize("N,K", [(1, 32), (17, 288), (16, 256), (40, 544), (33, 5120),
                                 (1000, 1312), (5, 17440)])
def test_tile_weight_matches_oracle(nv, orc, N, K):
    """Every byte of the tiled array, padding included."""
    import torch
    helpers.announce(f"tile_weight N={N} K={K}")
    rng = np.random.default_rng(N * 7 + K)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
    nbytes = nv.tiled_weight_bytes(N, K)
    assert nbytes == orc.tiled_weight_bytes(N, K)
    g = helpers.Guarded((nbytes,), torch.uint8)
    g.t.fill_(0xA5)  # every byte must be written
    nv.tile_weight(helpers.dev_u8(codes), helpers.dev_u8(scales), out=g.t)
    g.check()
    assert np.array_equal(g.t.cpu().numpy(), orc.tile_weight(codes, scales, N, K))


@pytest.mark.parametrize("N,K,n_rows", [(40, 544, 17), (1000, 1312, 333), (300, 5120, 300)])
def test_tile_rows_matches_oracle(nv, orc, N, K, n_rows):
    """A listed row subset tiled as its own matrix: the oracle's tiling of the
    gathered rows, byte for byte."""
    import torch
    helpers.announce(f"tile_weight rows N={N} K={K} n_rows={n_rows}")
    rng = np.random.default_rng(N + K + n_rows)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
    idx = np.sort(rng.choice(N, n_rows, replace=False)).astype(np.int32)
    if n_rows == N:
        idx = rng.permutation(N).astype(np.int32)  # any order, not only sorted
    g = helpers.Guarded((nv.tiled_weight_bytes(n_rows, K),), torch.uint8)
    g.t.fill_(0x5A)
    nv.tile_weight(helpers.dev_u8(codes), helpers.dev_u8(scales), row_idx=helpers.dev_i32(idx),
                   out=g.t)
    g.check()
    ref = orc.tile_weight(codes[idx], scales[idx], n_rows, K)
    assert np.array_equal(g.t.cpu().numpy(), ref)


@pytest.mark.parametrize("M,K,N", [
    (1, 32, 16), (1, 64, 5), (2, 288, 33), (3, 544, 100), (4, 1024, 560), (5, 2080, 48),
    (8, 1312, 300), (13, 256, 17), (16, 4096, 40), (17, 512, 48), (32, 1536, 272),
    (33, 768, 64), (40, 800, 90), (1, 17440, 200), (4, 8224, 24),
])
def test_ragged_shapes(nv, orc, M, K, N):
    """Shapes spanning several tiles with ragged tails in M, N (16-row tiles) and
    K (256-element steps, K % 32 == 0), bf16 and fp32 outputs."""
    helpers.announce(f"gemm_tiled ragged M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 1000 + N + 7)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    wt = _tiled(nv, w)
    _assert_close(_run(nv, x, wt, N), ref, what=f"{M}x{K}x{N}")
    _assert_close(_run(nv, x, wt, N, out_f32=True), ref, out_f32=True, what=f"{M}x{K}x{N} fp32")


# (M, plan): every built tiled layout -- the 4x4x4 kernel (M <= 8 with
# gemv_small_max) with 1 or 2 tiles per wave, the 16x16 kernel with 1, 2, 4
# tiles and 4, 8, 16 waves (8-row activation window for M <= 8), K parts
# across workgroups
LAYOUTS = [
    (1, dict(gemv_tiles=1, gemv_waves=4)), (1, dict(gemv_tiles=2, gemv_waves=8)),
    (3, dict(gemv_tiles=1, gemv_waves=2, gemv_splits=3)), (4, dict(gemv_tiles=2, gemv_waves=4)),
    (7, dict(gemv_small_max=8, gemv_tiles=1, gemv_waves=4)),
    (1, dict(gemv_small_max=0, gemv_tiles=2, gemv_waves=8)),
    (8, dict(gemv_tiles=1, gemv_waves=4)), (8, dict(gemv_tiles=2, gemv_waves=8, gemv_splits=5)),
    (11, dict(gemv_tiles=4, gemv_waves=4)), (6, dict(gemv_tiles=4, gemv_waves=4)),
    (7, dict(gemv_tiles=1, gemv_waves=8, gemv_splits=2)),
    (16, dict(gemv_tiles=2, gemv_waves=4, gemv_splits=1)),
    (20, dict(gemv_tiles=1, gemv_waves=16)), (32, dict(gemv_tiles=2, gemv_waves=16)),
    (32, dict(gemv_tiles=2, gemv_waves=8)), (25, dict(gemv_tiles=1, gemv_waves=4, gemv_splits=7)),
    (2, dict(gemv_tiles=1, gemv_waves=8, gemv_lds_kib=8)),
    # K parts inside the workgroup: the 4x4x4 kernel (1 tile per wave, nw = groups x parts)
    (1, dict(gemv_kparts=2, gemv_waves=4)), (1, dict(gemv_kparts=8, gemv_waves=16)),
    (4, dict(gemv_kparts=4, gemv_waves=8)), (3, dict(gemv_kparts=8, gemv_waves=8, gemv_splits=1)),
    (2, dict(gemv_kparts=2, gemv_waves=8, gemv_lds_kib=8)),
    # ... and the 16x16 kernel
    (8, dict(gemv_kparts=4, gemv_tiles=2, gemv_waves=8)),
    (6, dict(gemv_kparts=8, gemv_tiles=1, gemv_waves=16)),
    (5, dict(gemv_kparts=8, gemv_tiles=2, gemv_waves=8)),
    (16, dict(gemv_kparts=2, gemv_tiles=2, gemv_waves=8)),
    (13, dict(gemv_kparts=4, gemv_tiles=1, gemv_waves=16, gemv_splits=2)),
    (32, dict(gemv_kparts=2, gemv_tiles=1, gemv_waves=16)),
]


@pytest.mark.parametrize("M,plan", LAYOUTS)
def test_every_layout(nv, orc, M, plan):
    helpers.announce(f"gemm_tiled layout M={M} {plan}")
    K, N = 2336, 700  # 10 steps (the last one partial), 44 tiles (the last one partial)
    rng = np.random.default_rng(M + len(plan))
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    wt = _tiled(nv, w)
    _assert_close(_run(nv, x, wt, N, plan=plan), ref, what=f"M={M} {plan}")
    _assert_close(_run(nv, x, wt, N, out_f32=True, plan=plan), ref, out_f32=True,
                  what=f"M={M} {plan} fp32")


@pytest.mark.parametrize("M,plan", [(8, dict(gemv_tiles=2, gemv_waves=8)),
                                    (12, dict(gemv_tiles=1, gemv_waves=4, gemv_splits=3)),
                                    (32, dict(gemv_tiles=2, gemv_waves=16)),
                                    (24, dict(gemv_tiles=1, gemv_waves=16, gemv_splits=2))])
def test_bit_identical_to_row_major(nv, M, plan):
    """The 16x16 kernel on tiled weights adds the same products in the same order
    as on row-major weights: identical fp32 outputs for the same launch layout
    (K % 256 == 0 so the row-major kernel takes no masked tail)."""
    import torch
    helpers.announce(f"gemm_tiled vs row-major M={M} {plan}")
    K, N = 2048, 1000
    rng = np.random.default_rng(M)
    x = helpers.dev_bf16(workloads.normal_bf16(rng, M, K))
    w = workloads.nvfp4_weight(rng, N, K)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    row = nv.gemm(x, wc, ws, out_dtype=torch.float32, plan=dict(plan, gemv_small_max=0))
    til = nv.gemm_tiled(x, nv.tile_weight(wc, ws), N, out_dtype=torch.float32,
                        plan=dict(plan, gemv_small_max=0))
    assert torch.equal(row, til)


def test_activations_outside_fp16(nv, orc):
    """Activations that fp16 cannot hold exactly (restaged steps of the fp16
    path) and K tails, on tiled weights."""
    helpers.announce("gemm_tiled fp16 restage")
    M, K, N = 8, 1312, 200
    rng = np.random.default_rng(11)
    x = workloads.normal_bf16(rng, M, K)
    xf = helpers.bf16_bits_to_f64(x)
    xf[0, 3] = 98304.0            # 1.5 * 2^16: above fp16's range
    xf[5, 700] = 1.5 * 2.0 ** -18  # below 2^-17: not exact as an fp16 subnormal
    xf[7, 1300] = -71680.0         # -1.09375 * 2^16
    x = helpers.f64_to_bf16_bits_exact(xf)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    wt = _tiled(nv, w)
    for M2 in (8, 32):
        xx = np.concatenate([x] * (M2 // 8))
        rr = np.concatenate([ref] * (M2 // 8))
        _assert_close(_run(nv, xx, wt, N, out_f32=True), rr, out_f32=True, what=f"M={M2}")


@pytest.mark.parametrize("M", [5, 300])
def test_w4a4_codes(nv, orc, M):
    """NVFP4 activations (a_dtype NVFP4) on tiled weights: the GEMV (M = 5) and
    the MFMA GEMM (M = 300, a shared round) after the activations' dequantize
    pass."""
    import torch
    helpers.announce(f"gemm_tiled W4A4 codes M={M}")
    K, N = 1024, 300
    rng = np.random.default_rng(5 + M)
    x = workloads.normal_bf16(rng, M, K)
    ac, asc = nv.quantize(helpers.dev_bf16(x))
    w = workloads.nvfp4_weight(rng, N, K)
    y = nv.gemm_tiled(ac, _tiled(nv, w), N, a_scales=asc, out_dtype=torch.float32)
    ref = orc.gemm_w4a4(ac.cpu().numpy(), asc.cpu().numpy(), M, K, w.codes, w.scales)
    _assert_close(y.cpu().numpy(), ref, out_f32=True, what="w4a4")


@pytest.mark.parametrize("K,N", workloads.DECODE_SHAPES)
def test_decode_full_size_sampled(nv, orc, K, N):
    """The decode shapes at full size on tiled weights for M in {1, 8, 32}, in
    the launch configuration the benchmark times; 512 sampled output columns
    recomputed by the oracle."""
    import torch
    w = workloads.decode_weights(K, N)
    wt = _tiled(nv, w)
    cols = np.sort(np.random.default_rng(K + N).choice(N, 512, replace=False)).astype(np.int32)
    ref_all = {}
    for M in workloads.DECODE_M:
        helpers.announce(f"gemm_tiled decode full size K={K} N={N} M={M}")
        x = workloads.decode_activations(M, K)
        y = helpers.host_bits(nv.gemm_tiled(helpers.dev_bf16(x), wt, N))
        ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=cols)
        _assert_close(y[:, cols], ref, what=f"K={K} N={N} M={M}")
        ref_all[M] = y
        torch.cuda.synchronize()
    # run to run: the same call again gives the same bits
    x = workloads.decode_activations(32, K)
    y2 = helpers.host_bits(nv.gemm_tiled(helpers.dev_bf16(x), wt, N))
    assert np.array_equal(y2, ref_all[32])


def test_masked_head_rows_tiled_full_size_sampled(nv, orc):
    """The masked head's 32,768 of 248,320 rows tiled once (row_idx) and streamed
    as a dense 32,768-row layer, M in {1, 8, 32}; sampled output columns against
    the oracle's masked product."""
    import torch
    K, N = workloads.HIDDEN, workloads.VOCAB
    w = workloads.decode_weights(K, N)
    idx = workloads.decode_masked_rows()
    wt = nv.tile_weight(helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                        row_idx=helpers.dev_i32(idx))
    sel = np.sort(np.random.default_rng(3).choice(len(idx), 256, replace=False))
    for M in workloads.DECODE_M:
        helpers.announce(f"gemm_tiled masked head rows M={M}")
        x = workloads.decode_activations(M, K)
        y = helpers.host_bits(nv.gemm_tiled(helpers.dev_bf16(x), wt, len(idx)))
        ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx[sel])
        _assert_close(y[:, sel], ref, what=f"masked M={M}")
        torch.cuda.synchronize()


# ---- the MFMA GEMM on tiled weights (M >= 65) ------------------------------------------

@pytest.mark.parametrize("M,K,N", [(65, 256, 40), (300, 1312, 700), (512, 2080, 272),
                                   (1000, 4096, 1000), (2048, 544, 5000)])
def test_mfma_tiled_matches_oracle(nv, orc, M, K, N):
    """Ragged M, N (partial 256 x 256 tiles and 16-row weight tiles), K % 64 == 32
    and K % 256 != 0, whole and shared rounds; every output against the oracle,
    guarded; fp32 outputs identical to the row-major MFMA GEMM (same partition,
    same products in the same order)."""
    import torch
    helpers.announce(f"gemm_tiled mfma M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    wt = _tiled(nv, w)
    _assert_close(_run(nv, x, wt, N), ref, what=f"{M}x{K}x{N}")
    got = _run(nv, x, wt, N, out_f32=True)
    _assert_close(got, ref, out_f32=True, what=f"{M}x{K}x{N} fp32")
    row = nv.gemm(helpers.dev_bf16(x), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                  out_dtype=torch.float32)
    assert np.array_equal(row.cpu().numpy(), got)


def test_mfma_tiled_prefill_full_size_sampled(nv, orc):
    """Prefill M = 8192, K = 5120, N = 17408 on tiled weights: 256 sampled rows x
    all columns against the oracle."""
    helpers.announce("gemm_tiled prefill 8192x5120x17408")
    M, K, N = 8192, workloads.HIDDEN, workloads.MLP
    x, w = workloads.prefill(K, N)
    wt = _tiled(nv, w)
    y = helpers.host_bits(nv.gemm_tiled(helpers.dev_bf16(x), wt, N))
    rows = np.sort(np.random.default_rng(9).choice(M, 64, replace=False))
    ref = orc.gemm_w4a16(x[rows], len(rows), K, w.codes, w.scales)
    _assert_close(y[rows], ref, what="prefill tiled")


# ---- grouped GEMMs on tiled expert weights -----------------------------------------------

def _grouped_case(rng, E, K, N, counts, rows):
    counts = np.array(counts)
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = workloads.normal_bf16(rng, rows, K)
    w = workloads.nvfp4_weight(rng, E, N, K)
    gather = rng.integers(0, rows, R).astype(np.int32)
    rs = (rng.random(R) + 0.5).astype(np.float32)
    return R, off, a, w, gather, rs


@pytest.mark.parametrize("mfma", [False, True])
@pytest.mark.parametrize("epi,scaled", [(0, False), (1, False), (0, True), (1, True)])
def test_grouped_tiled(nv, orc, mfma, epi, scaled):
    """Both grouped kernels on tiled experts (the MFMA one forced through the
    plan), both epilogues, single- and two-level experts, uneven groups (empty,
    one row, several chunks), K % 256 != 0: against the oracle, guarded, and
    bit-identical to the row-major call of the same kernel."""
    helpers.announce(f"grouped tiled mfma={mfma} epi={epi} scaled={scaled}")
    rng = np.random.default_rng(7 + 2 * epi + scaled + 4 * mfma)
    E, K, N = 6, 544 if not mfma else 416, 96 if not mfma else 352
    counts = [0, 1, 40, 0, 70, 9] if not mfma else [0, 1, 300, 256, 600, 37]
    R, off, a, w, gather, rs = _grouped_case(rng, E, K, N, counts, 120)
    gs = (2.0 ** rng.integers(-3, 4, E) * (1 + rng.random(E))).astype(np.float32) if scaled else None
    plan = {"grouped_mfma_min_rows": 1} if mfma else {"grouped_mfma_min_rows": 1 << 20,
                                                       "grouped_gemv_waves": 4 << (epi + scaled)}
    wc, wsc = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    wt = nv.tile_experts(wc, wsc)
    kw = dict(row_scale=helpers.dev_f32(rs), epilogue=epi, plan=plan,
              w_global=None if gs is None else helpers.dev_f32(gs))
    g = helpers.Guarded((R, N // 2 if epi else N), torch.bfloat16)
    y = nv.grouped_gemm_tiled(helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
                              wt, E, N, R, out=g.t, **kw)
    g.check()
    ref = orc.grouped_gemm(a, K, gather, off, E, R, N, w.codes, w.scales, row_scale=rs,
                           epilogue=epi, w_global=gs)
    ok, rf, worst = helpers.gemm_close(helpers.host_bits(y), ref)
    assert ok, (rf, worst)
    yr = nv.grouped_gemm(helpers.dev_bf16(a), helpers.dev_i32(gather), helpers.dev_i32(off),
                         wc, wsc, R, **kw)
    assert torch.equal(y, yr)


@pytest.mark.parametrize("T", [32, 4096])
def test_moe_layer_tiled_equals_row_major(nv, T):
    """The routed layer (hidden 2048, 128 experts, top-8, expert intermediate
    768) on tiled experts gives the row-major layer's output bit for bit (the
    row-major layer is checked against the oracle in test_gpu_moe.py)."""
    helpers.announce(f"moe layer tiled T={T}")
    m = workloads.moe(T)
    E, I = 128, m.w2.codes.shape[2] * 2
    args = (helpers.dev_bf16(m.x), helpers.dev_i32(m.ids), helpers.dev_f32(m.gates))
    w1c, w1s = helpers.dev_u8(m.w1.codes), helpers.dev_u8(m.w1.scales)
    w2c, w2s = helpers.dev_u8(m.w2.codes), helpers.dev_u8(m.w2.scales)
    row = nv.moe_layer(*args, w1c, w1s, w2c, w2s)
    til = nv.moe_layer_tiled(*args, nv.tile_experts(w1c, w1s), nv.tile_experts(w2c, w2s), E, I)
    assert torch.equal(row, til)
