"""GPU parity of nvfp4_gemm (W4A16 and W4A4, full and masked rows) against the
fp64 oracle.  Tolerance: relative Frobenius error <= 1e-3 and every element
within 1e-2*(|ref|+1), against the oracle rounded once to bf16 for bf16 outputs
and unrounded for fp32 outputs."""
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


def _plan(spec):
    """"tiles,waves[,lds_kib[,splits]]" -> a GEMV plan override (None: default)."""
    if spec is None:
        return None
    keys = ("gemv_tiles", "gemv_waves", "gemv_lds_kib", "gemv_splits")
    return {k: int(v) for k, v in zip(keys, spec.split(",")) if int(v) > 0}


def _run(nv, x, w, row_idx=None, out_f32=False, plan=None):
    """The product on the GPU into a guard-padded output (a write outside the
    output fails the case)."""
    import torch
    xd = helpers.dev_bf16(x)
    ri = None if row_idx is None else helpers.dev_i32(row_idx)
    dt = torch.float32 if out_f32 else torch.bfloat16
    n_out = w.codes.shape[0] if row_idx is None else len(row_idx)
    g = helpers.Guarded((x.shape[0], n_out), dt)
    y = nv.gemm(xd, helpers.dev_u8(w.codes), helpers.dev_u8(w.scales), row_idx=ri,
                out_dtype=dt, plan=plan, out=g.t)
    g.check()
    return y.cpu().numpy() if out_f32 else helpers.host_bits(y)


def _assert_close(got, ref, out_f32=False, what=""):
    ok, rf, worst = helpers.gemm_close(got, ref, out_is_bf16=not out_f32)
    assert ok, f"{what}: rel_frob={rf:.3e} worst_elem_ratio={worst:.3f}"
    return rf


def test_tiny_config(nv, orc):
    """M=1, K=512, N=1024 -- the tiny seeded workload, bf16 and fp32 outputs."""
    helpers.announce("gemm tiny M=1 K=512 N=1024")
    x, w = workloads.tiny()
    ref = orc.gemm_w4a16(x, 1, 512, w.codes, w.scales)
    _assert_close(_run(nv, x, w), ref, what="tiny bf16")
    rf = _assert_close(_run(nv, x, w, out_f32=True), ref, out_f32=True, what="tiny fp32")
    assert rf < 1e-5


@pytest.mark.parametrize("M,K,N", [
    (1, 32, 16), (1, 64, 5), (3, 288, 33), (8, 1024, 560), (16, 2080, 100), (17, 512, 48),
    (32, 1536, 272), (33, 768, 64), (70, 256, 40), (5, 8192, 24), (6, 1312, 300),
    (7, 544, 33000), (4, 8192, 24), (4, 8224, 40), (1, 17440, 200),
])
def test_ragged_shapes(nv, orc, M, K, N):
    """Shapes spanning several tiles with ragged tails in M (16-row MFMA tiles),
    N (16-row weight tiles), and K (256-element steps, K % 32 == 0)."""
    helpers.announce(f"gemm ragged M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 1000 + N)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    _assert_close(_run(nv, x, w), ref, what=f"{M}x{K}x{N}")
    _assert_close(_run(nv, x, w, out_f32=True), ref, out_f32=True, what=f"{M}x{K}x{N} fp32")


@pytest.mark.parametrize("plan", ["2,16", "1,16", "2,8", "1,4"])
@pytest.mark.parametrize("M,K,N", [(17, 2048, 700), (32, 1312, 1000), (24, 4096, 1100),
                                   (32, 256, 33)])
def test_two_tiles_plans(nv, orc, M, K, N, plan):
    """Two activation tiles (16 < M <= 32) in every workgroup layout, forced
    through a plan ("tiles per wave, waves") at sizes the oracle checks whole:
    16-wave workgroups (the fp16 path, scale blocks for K % 256 == 0) and the
    8- and 4-wave bf16 layouts; ragged M, N and K, waves with padding rows
    only."""
    helpers.announce(f"gemm two tiles 16 waves M={M} K={K} N={N} plan={plan}")
    rng = np.random.default_rng(M * 7 + K + N)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    got = _run(nv, x, w, plan=_plan(plan))
    got32 = _run(nv, x, w, out_f32=True, plan=_plan(plan))
    _assert_close(got, ref, what=f"{M}x{K}x{N}")
    _assert_close(got32, ref, out_f32=True, what=f"{M}x{K}x{N} fp32")


def test_identity_activations_reproduce_weights(nv, orc):
    """x = one-hot rows: y[m][n] = w[n][k_m] exactly (a single exact product), so
    the GEMV's in-register dequantization is checked bit-exactly against the
    oracle's dequantization (zero signs aside)."""
    helpers.announce("gemm identity activations")
    K, N = 1024, 96
    w = workloads.nvfp4_weight(np.random.default_rng(9), N, K)
    ks = np.array([0, 1, 15, 16, 31, 32, 127, 128, 255, 256, 511, 512, 777, 1000, 1022, 1023,
                   3, 64, 200, 300, 400, 500, 600, 700, 800, 900, 33, 34, 35, 36, 37, 38])
    M = len(ks)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80  # 1.0
    got = _run(nv, x, w)
    deq = orc.dequantize(w.codes, w.scales, N, K)
    want = deq[:, ks].T
    assert np.array_equal(got & 0x7FFF, want & 0x7FFF)
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz])


def test_masked_rows(nv, orc):
    helpers.announce("gemm masked rows")
    rng = np.random.default_rng(10)
    M, K, N = 8, 512, 4000
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, 333, replace=False)).astype(np.int32)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx)
    _assert_close(_run(nv, x, w, row_idx=idx), ref, what="masked")
    # degenerate: a single kept row, and every row kept through row_idx
    one = np.array([N - 1], np.int32)
    _assert_close(_run(nv, x, w, row_idx=one),
                  orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=one), what="one row")
    allr = np.arange(N, dtype=np.int32)
    _assert_close(_run(nv, x, w, row_idx=allr), orc.gemm_w4a16(x, M, K, w.codes, w.scales),
                  what="all rows via idx")


def test_zero_and_extreme_weights(nv, orc):
    """All-zero codes give exact zeros; maximal scales (448) with +-6 codes and
    outlier activations stay within tolerance (|w| = 2688)."""
    helpers.announce("gemm zero / extreme weights")
    import torch
    M, K, N = 4, 512, 64
    x = workloads.normal_bf16(np.random.default_rng(11), M, K, outlier_frac=0.02)
    w = workloads.NF4W(np.zeros((N, K // 2), np.uint8), np.full((N, K // 16), 0x7E, np.uint8))
    assert np.all((_run(nv, x, w) & 0x7FFF) == 0)
    w = workloads.NF4W(np.full((N, K // 2), 0xF7, np.uint8), np.full((N, K // 16), 0x7E, np.uint8))
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    _assert_close(_run(nv, x, w), ref, what="extreme")


@pytest.mark.parametrize("M,plan", [(8, None), (32, None), (32, "2,16"), (20, "2,8")])
def test_activations_outside_fp16(nv, orc, M, plan):
    """Steps whose activations are not all exact in fp16 (values beyond its
    range, below its precision, or bf16 subnormals) take the bf16 path of the
    16x16 GEMV, the other steps the fp16 path; with a failing value in every
    step the workgroups stop converting after two.  The product stays within
    the GEMM tolerance either way, with both K layouts (scale blocks and K
    tail).  plan ("tiles,waves" of the GEMV plan): "2,16" two weight tiles
    per wave in 16-wave workgroups (the widest layers at M > 16), "2,8" the
    8-wave bf16 layout."""
    helpers.announce(f"gemm activations outside fp16 M={M} plan={plan}")
    _outside_fp16_cases(nv, orc, M, _plan(plan))


def _outside_fp16_cases(nv, orc, M, plan):
    rng = np.random.default_rng(40 + M)
    for K, N in ((2048, 700), (1312, 260)):
        x = workloads.normal_bf16(rng, M, K)
        x[0, 300] = 0x4880          # 2^18: beyond fp16's range
        x[M - 1, 1000] = 0x3380     # 2^-24 * 1.0: below fp16's precision for 8 bits
        x[M // 2, 1030] = 0x0005    # a bf16 subnormal
        x[1, 5] = 0xC780            # -65536: rounds to fp16 infinity
        if K == 2048:               # every step fails: workgroups switch to bf16 for good
            x[2, ::256] = 0x3380
        w = workloads.nvfp4_weight(rng, N, K)
        ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
        _assert_close(_run(nv, x, w, plan=plan), ref, what=f"{M}x{K}x{N} bf16 steps")
        _assert_close(_run(nv, x, w, out_f32=True, plan=plan), ref, out_f32=True,
                      what=f"{M}x{K}x{N} fp32")


@pytest.mark.parametrize("K,N", workloads.DECODE_SHAPES)
def test_decode_full_size_sampled(nv, orc, K, N):
    """The decode shapes at full size for M in {1, 8, 32}, in the launch
    configuration the benchmark times; 512 output columns sampled per M are
    recomputed by the oracle (whole rows of W, all M rows of x)."""
    import torch
    w = workloads.decode_weights(K, N)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    cols = np.sort(np.random.default_rng(K + N).choice(N, 512, replace=False)).astype(np.int32)
    for M in workloads.DECODE_M:
        helpers.announce(f"gemm decode full size K={K} N={N} M={M}")
        x = workloads.decode_activations(M, K)
        y = helpers.host_bits(nv.gemm(helpers.dev_bf16(x), wc, ws))
        ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=cols)
        _assert_close(y[:, cols], ref, what=f"K={K} N={N} M={M}")
        torch.cuda.synchronize()


def test_masked_head_full_size_sampled(nv, orc):
    """Masked head: 32,768 of 248,320 rows, K = 5120, M in {1, 8, 32}; sampled
    output columns against the oracle."""
    import torch
    K, N = workloads.HIDDEN, workloads.VOCAB
    w = workloads.decode_weights(K, N)
    idx = workloads.decode_masked_rows()
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    sel = np.sort(np.random.default_rng(3).choice(len(idx), 256, replace=False))
    for M in workloads.DECODE_M:
        helpers.announce(f"gemm masked head M={M}")
        x = workloads.decode_activations(M, K)
        xd = helpers.dev_bf16(x)
        y = helpers.host_bits(nv.gemm(xd, wc, ws, row_idx=helpers.dev_i32(idx)))
        ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx[sel])
        _assert_close(y[:, sel], ref, what=f"masked M={M}")
        torch.cuda.synchronize()


def test_w4a4_gemm(nv, orc):
    """W4A4: quantize the 512 x 5120 activations on the GPU, then GEMM against
    NF4W(17408, 5120); sampled columns against the oracle's W4A4 on the oracle's
    (bit-identical) codes."""
    helpers.announce("gemm W4A4 512x5120 -> 17408")
    x, w = workloads.w4a4()
    gc, gs = nv.quantize(helpers.dev_bf16(x))
    rc, rs = orc.quantize(x, 512, 5120)
    assert np.array_equal(gc.cpu().numpy(), rc) and np.array_equal(gs.cpu().numpy(), rs)
    y = helpers.host_bits(nv.gemm(gc, helpers.dev_u8(w.codes), helpers.dev_u8(w.scales),
                                  a_scales=gs))
    cols = np.sort(np.random.default_rng(4).choice(17408, 256, replace=False)).astype(np.int32)
    ref = orc.gemm_w4a4(rc, rs, 512, 5120, w.codes, w.scales, row_idx=cols)
    _assert_close(y[:, cols], ref, what="w4a4")


def test_run_to_run_bit_identical(nv):
    """Fixed reduction order: two runs of a split-K shape give the same bits."""
    helpers.announce("gemm determinism")
    rng = np.random.default_rng(12)
    M, K, N = 32, 17408, 1024
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    a = _run(nv, x, w)
    b = _run(nv, x, w)
    assert np.array_equal(a, b)


# ---- large M: the LDS-tiled MFMA GEMM (256 x 256 tiles, 64-element K steps) ----

@pytest.mark.parametrize("M,K,N", [
    (65, 64, 16),       # smallest M on the MFMA path, one K step
    (300, 160, 520),    # ragged in every dimension; K % 64 == 32 (partial and padding steps)
    (257, 96, 257),     # N % 4 != 0: element-wise epilogue
    (512, 5120, 300),   # long K
    (1000, 1088, 777),  # several tiles in M and N, ragged tails (split-K: 2 parts)
    (300, 2080, 300),   # split-K in 4 parts, the last ending on a partial K step
])
def test_mfma_ragged_shapes(nv, orc, M, K, N):
    helpers.announce(f"gemm mfma ragged M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 7 + N + K)
    x = workloads.normal_bf16(rng, M, K, outlier_frac=0.01)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    _assert_close(_run(nv, x, w), ref, what=f"{M}x{K}x{N}")
    _assert_close(_run(nv, x, w, out_f32=True), ref, out_f32=True, what=f"{M}x{K}x{N} fp32")


def test_mfma_identity_activations_reproduce_weights(nv, orc):
    """One-hot activation rows through the MFMA path: y[m][n] = w[n][k_m], the
    LDS-staged dequantization compared bit for bit with the oracle's."""
    helpers.announce("gemm mfma identity activations")
    K, N, M = 1056, 300, 300
    w = workloads.nvfp4_weight(np.random.default_rng(19), N, K)
    ks = np.random.default_rng(20).integers(0, K, M)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80  # 1.0
    got = _run(nv, x, w)
    want = orc.dequantize(w.codes, w.scales, N, K)[:, ks].T
    assert np.array_equal(got & 0x7FFF, want & 0x7FFF)
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz])


def test_mfma_masked_rows(nv, orc):
    helpers.announce("gemm mfma masked rows")
    rng = np.random.default_rng(21)
    M, K, N = 300, 512, 4000
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, 333, replace=False)).astype(np.int32)
    _assert_close(_run(nv, x, w, row_idx=idx),
                  orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx), what="masked")
    one = np.array([7], np.int32)
    _assert_close(_run(nv, x, w, row_idx=one),
                  orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=one), what="one row")


def test_mfma_matches_gemv_chunks(nv):
    """The same product through both paths (the plan's gemm_min_m forces the
    GEMV at M = 96): both are fp32 sums of exact products, so they agree to
    fp32 rounding."""
    helpers.announce("gemm mfma vs gemv")
    rng = np.random.default_rng(22)
    M, K, N = 96, 2048, 512
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    a = _run(nv, x, w, out_f32=True)
    b = _run(nv, x, w, out_f32=True, plan={"gemm_min_m": 100000})
    scale = np.abs(a).max() + 1.0
    assert np.max(np.abs(a - b)) <= 1e-5 * scale


@pytest.mark.parametrize("M,K,N", [(300, 160, 520), (700, 2048, 1000)])
def test_mfma_w4a4_ragged(nv, orc, M, K, N):
    helpers.announce(f"gemm mfma w4a4 M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    x = workloads.normal_bf16(rng, M, K, outlier_frac=0.01)
    w = workloads.nvfp4_weight(rng, N, K)
    rc, rs = orc.quantize(x, M, K)
    y = helpers.host_bits(nv.gemm(helpers.dev_u8(rc), helpers.dev_u8(w.codes),
                                  helpers.dev_u8(w.scales), a_scales=helpers.dev_u8(rs)))
    _assert_close(y, orc.gemm_w4a4(rc, rs, M, K, w.codes, w.scales), what="w4a4")



@pytest.mark.parametrize("M,K,N,shared", [(300, 3136, 712, True), (1300, 2560, 12808, False)])
def test_mfma_split_tiles_partial_last_column_tile(nv, orc, M, K, N, shared):
    """Split tiles whose last column tile is partial with N % 8 == 0, so the
    reduce stores whole 8-column runs up to the edge: a shared round (6 tiles)
    and a split last round (306 tiles: 50 split, the last 8 columns wide).
    bf16 and fp32 outputs, guarded; columns around every tile edge against the
    oracle (all of them for the shared round)."""
    helpers.announce(f"gemm mfma split tiles partial column tile M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N + 5)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    if shared:
        cols = np.arange(N, dtype=np.int32)
    else:
        edges = np.arange(0, N + 1, 256)
        cols = np.unique(np.clip(np.concatenate([edges - 1, edges, edges + 7, [N - 8, N - 1]]),
                                 0, N - 1)).astype(np.int32)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=cols)
    _assert_close(_run(nv, x, w)[:, cols], ref, what="bf16")
    _assert_close(_run(nv, x, w, out_f32=True)[:, cols], ref, out_f32=True, what="fp32")


def test_mfma_tail_tiles_split(nv, orc):
    """300 tiles on 256 CUs: the first 256 run whole, the last 44 (columns
    10752 .. 12796 in the tile order) run as 5 K parts summed by the reduce
    kernel.  Ragged M and N (N % 4 != 0); all rows, 384 columns (160 of them in
    the split tiles, including the last) against the oracle."""
    import torch
    M, K, N = 1300, 2560, 12797
    helpers.announce(f"gemm mfma tail split M={M} K={K} N={N}")
    rng = np.random.default_rng(77)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    y = helpers.host_bits(nv.gemm(helpers.dev_bf16(x), helpers.dev_u8(w.codes),
                                  helpers.dev_u8(w.scales)))
    cols = np.unique(np.concatenate([rng.choice(10752, 222, replace=False),
                                     rng.choice(np.arange(10752, N), 158, replace=False),
                                     [0, 10751, 10752, N - 1]])).astype(np.int32)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=cols)
    _assert_close(y[:, cols], ref, what="tail split")
    torch.cuda.synchronize()

@pytest.mark.parametrize("M,K,N,slots", [(256, 5120, 256, 8), (300, 3136, 700, 6),
                                         (512, 5120, 1100, 8), (65, 2080, 4100, 5)])
def test_mfma_shared_round(nv, orc, M, K, N, slots):
    """Fewer 256 x 256 tiles than CUs: every tile is shared by one round of
    workgroups, each taking an equal range of all the tiles' K steps -- the end
    of one tile and the start of the next -- summed per tile in K order by the
    reduce (`slots` = most segments of one tile, read off the workspace size).
    One tile in 8 segments, ragged tiles and N, a partial last K step
    (K % 64 == 32); every output against the oracle, guarded output, run-to-run
    bit-identical, and the fused W4A4 tile loads bit-identical to quantize + the
    W4A4 GEMM on the same partition."""
    import torch
    helpers.announce(f"gemm mfma shared round M={M} K={K} N={N}")
    tiles = -(-M // 256) * -(-N // 256)
    assert nv.gemm_workspace_size(M, N, K, N) == tiles * slots * 256 * 256 * 4
    rng = np.random.default_rng(M + K + N)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    y = _run(nv, x, w, out_f32=True)
    _assert_close(y, orc.gemm_w4a16(x, M, K, w.codes, w.scales), out_f32=True, what="shared")
    assert np.array_equal(y.view(np.int32), _run(nv, x, w, out_f32=True).view(np.int32))
    xd, wc, ws = helpers.dev_bf16(x), helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    fused = nv.gemm_w4a4(xd, wc, ws, out_dtype=torch.float32, plan={"w4a4_fuse": 1})
    ac, as_ = nv.quantize(xd)
    ref = nv.gemm(ac, wc, ws, a_scales=as_, out_dtype=torch.float32)
    assert torch.equal(fused.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("K,N", [(5120, 17408), (17408, 5120)])
def test_prefill_full_size_sampled(nv, orc, K, N):
    """The prefill shapes at full size (M = 8192, outlier activations), in the
    launch configuration the benchmark times; 48 rows x 256 columns sampled are
    recomputed by the oracle."""
    import torch
    helpers.announce(f"gemm prefill full size M=8192 K={K} N={N}")
    x, w = workloads.prefill(K, N)
    y = helpers.host_bits(nv.gemm(helpers.dev_bf16(x), helpers.dev_u8(w.codes),
                                  helpers.dev_u8(w.scales)))
    sr = np.random.default_rng(K)
    rows = np.sort(np.concatenate([sr.choice(8192, 46, replace=False), [0, 8191]]))
    rows = np.unique(rows)
    cols = np.sort(np.concatenate([sr.choice(N, 254, replace=False), [0, N - 1]]))
    cols = np.unique(cols).astype(np.int32)
    xs = np.ascontiguousarray(x[rows])
    ref = orc.gemm_w4a16(xs, len(rows), K, w.codes, w.scales, row_idx=cols)
    _assert_close(y[np.ix_(rows, cols)], ref, what=f"prefill K={K} N={N}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,plan", [(1, "2,4,0,8"), (1, "2,4,0,11"), (8, "2,4,0,8"),
                                    (8, "2,8,0,16"), (32, "1,16,0,11"), (32, "2,16,0,16"),
                                    (3, "1,4,0,13")])
def test_split_k_part_counts(nv, orc, M, plan):
    """K split into 8, 11, 13 and 16 parts (plan "tiles,waves,lds,splits"): the
    reduce adds full batches of eight parts and every remainder; bf16 and
    fp32 outputs within the GEMM tolerance of the oracle."""
    helpers.announce(f"gemm split-K part counts M={M} plan={plan}")
    rng = np.random.default_rng(M * 11 + len(plan))
    K, N = 8192, 300
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    got = _run(nv, x, w, plan=_plan(plan))
    got32 = _run(nv, x, w, out_f32=True, plan=_plan(plan))
    _assert_close(got, ref, what=f"{M}x{K}x{N} {plan}")
    _assert_close(got32, ref, out_f32=True, what=f"{M}x{K}x{N} {plan} fp32")


KP_LAYOUTS = [(2, 8, 4), (2, 8, 2), (1, 16, 4), (1, 8, 2), (2, 16, 8), (1, 16, 8), (2, 8, 8)]


@pytest.mark.parametrize("tiles,waves,parts", KP_LAYOUTS)
@pytest.mark.parametrize("M,K,N", [(8, 2304, 700), (5, 4352, 333), (16, 1280, 1000),
                                   (7, 5120, 40)])
def test_kparts_layouts(nv, orc, M, K, N, tiles, waves, parts):
    """K parts inside the workgroup (plan gemv_kparts): every built layout, part
    lengths that do not divide the K steps evenly, ragged N (padding columns),
    one to sixteen activation rows; bf16 and fp32 outputs within the GEMM
    tolerance of the oracle, guarded outputs."""
    if parts == 8 and M > 8:
        pytest.skip("eight parts are built for 8-row windows (M <= 8) only")
    helpers.announce(f"gemm kparts M={M} K={K} N={N} layout={tiles},{waves},{parts}")
    rng = np.random.default_rng(M * 3 + K + N + parts)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    plan = {"gemv_tiles": tiles, "gemv_waves": waves, "gemv_kparts": parts}
    _assert_close(_run(nv, x, w, plan=plan), ref, what=f"{M}x{K}x{N}")
    _assert_close(_run(nv, x, w, out_f32=True, plan=plan), ref, out_f32=True,
                  what=f"{M}x{K}x{N} fp32")


@pytest.mark.parametrize("M,K,N", [(32, 2304, 700), (17, 4352, 333), (24, 512, 40)])
def test_kparts_two_tiles(nv, orc, M, K, N):
    """K parts with two activation tiles (1 tile per wave, 16 waves, 2 parts):
    ragged M, N and part lengths; bf16 and fp32 outputs against the oracle."""
    helpers.announce(f"gemm kparts two tiles M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + 5 * N)
    x = workloads.normal_bf16(rng, M, K)
    w = workloads.nvfp4_weight(rng, N, K)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales)
    plan = {"gemv_tiles": 1, "gemv_waves": 16, "gemv_kparts": 2}
    _assert_close(_run(nv, x, w, plan=plan), ref, what=f"{M}x{K}x{N}")
    _assert_close(_run(nv, x, w, out_f32=True, plan=plan), ref, out_f32=True,
                  what=f"{M}x{K}x{N} fp32")


@pytest.mark.parametrize("tiles,waves,parts", [(2, 8, 4), (1, 16, 8)])
def test_kparts_masked_outside_fp16_and_splits(nv, orc, tiles, waves, parts):
    """K parts with a row mask, activations outside fp16 in some steps (the
    whole window buffer is restaged in bf16 and the workgroup stops converting
    after two), and K parts across workgroups as well (plan gemv_splits): the
    fp32 partials of each workgroup are its parts' sum."""
    helpers.announce(f"gemm kparts masked/outside fp16/splits layout={tiles},{waves},{parts}")
    rng = np.random.default_rng(77 + parts)
    M, K, N = 8, 4096, 3000
    x = workloads.normal_bf16(rng, M, K)
    x[0, 300] = 0x4880          # 2^18: beyond fp16's range
    x[3, 1500] = 0x3380         # below fp16's precision for 8 bits
    x[7, 4000] = 0x0005         # a bf16 subnormal
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, 777, replace=False)).astype(np.int32)
    ref = orc.gemm_w4a16(x, M, K, w.codes, w.scales, row_idx=idx)
    for z in (None, 2):
        plan = {"gemv_tiles": tiles, "gemv_waves": waves, "gemv_kparts": parts}
        if z:
            plan["gemv_splits"] = z
        _assert_close(_run(nv, x, w, row_idx=idx, plan=plan), ref, what=f"masked z={z}")
    x2 = x.copy()
    x2[1, ::256] = 0x3380       # every step: workgroups switch to bf16 for good
    ref2 = orc.gemm_w4a16(x2, M, K, w.codes, w.scales)
    _assert_close(_run(nv, x2, w, out_f32=True,
                       plan={"gemv_tiles": tiles, "gemv_waves": waves, "gemv_kparts": parts}),
                  ref2, out_f32=True, what="every step restaged")
