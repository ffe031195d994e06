"""The C ABI without a GPU: the library loads, exports every function that
include/nvfp4.h declares, and rejects invalid arguments on the host with the
documented status codes before making any HIP call."""
import ctypes
import os
import re

import pytest

import bit_quantized_gemm_nvfp4_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

SUCCESS, INVALID, NOT_SUPPORTED, WORKSPACE, LAUNCH = 0, 1, 2, 3, 4

# fake, 256-byte aligned "device" addresses: validation must fail before any use
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
P4 = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10008)  # 8-byte aligned only
NULL = None


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.library_path()):
        import bit_quantized_gemm_nvfp4_amd.build as b
        b.build()
    return nv.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
        assert n in nv._SIGS, f"binding misses {n}"


def test_status_strings(L):
    for s in range(5):
        assert L.nvfp4_status_string(s).decode().startswith("NVFP4")
    assert b"unknown" in L.nvfp4_status_string(99)
    assert L.nvfp4_version() >= 100


def test_dequantize_validation(L):
    assert L.nvfp4_dequantize(NULL, P2, 4, 64, P3, NULL) == INVALID
    assert L.nvfp4_dequantize(P, P2, 0, 64, P3, NULL) == INVALID
    assert L.nvfp4_dequantize(P, P2, 4, 48, P3, NULL) == NOT_SUPPORTED
    assert L.nvfp4_dequantize(MIS, P2, 4, 64, P3, NULL) == INVALID


def test_quantize_validation(L):
    assert L.nvfp4_quantize(P, 4, 64, NULL, P3, NULL) == INVALID
    assert L.nvfp4_quantize(P, -1, 64, P2, P3, NULL) == INVALID
    assert L.nvfp4_quantize(P, 4, 40, P2, P3, NULL) == NOT_SUPPORTED
    assert L.nvfp4_quantize(P, 4, 64, P2, MIS, NULL) == INVALID


def _gemm(L, a_dtype=0, a=P, a_scales=NULL, M=4, N=64, K=256, wc=P2, ws=P3, row_idx=NULL,
          n_out=64, out_dtype=0, out=P4, workspace=NULL, wbytes=0):
    return L.nvfp4_gemm(a_dtype, a, a_scales, M, N, K, wc, ws, row_idx, n_out, out_dtype, out,
                        workspace, wbytes, NULL)


def test_gemm_validation(L):
    assert _gemm(L, a=NULL) == INVALID
    assert _gemm(L, M=0) == INVALID
    assert _gemm(L, K=48) == NOT_SUPPORTED
    assert _gemm(L, a_dtype=7) == NOT_SUPPORTED
    assert _gemm(L, out_dtype=2) == NOT_SUPPORTED
    assert _gemm(L, a_scales=P) == INVALID             # bf16 activations take no scales
    assert _gemm(L, a_dtype=2) == INVALID              # NVFP4 activations need scales
    assert _gemm(L, n_out=32) == INVALID               # no row_idx: n_out must be N
    assert _gemm(L, row_idx=P, n_out=65) == INVALID    # more rows than N
    assert _gemm(L, wc=MIS) == INVALID
    # a shape that needs workspace, given none
    need = L.nvfp4_gemm_workspace_size(0, 32, 5120, 17408, 5120)
    assert need > 0
    assert _gemm(L, M=32, N=5120, K=17408, n_out=5120) == WORKSPACE
    assert _gemm(L, M=32, N=5120, K=17408, n_out=5120, workspace=P, wbytes=need - 1) == WORKSPACE



def _w4a4(L, a=P, M=4, N=64, K=256, wc=P2, ws=P3, row_idx=NULL, n_out=64, out_dtype=0, out=P4,
          workspace=NULL, wbytes=0):
    return L.nvfp4_gemm_w4a4_bf16(a, M, N, K, wc, ws, row_idx, n_out, out_dtype, out, workspace,
                                  wbytes, NULL)


def test_gemm_w4a4_bf16_validation(L):
    """Every argument is checked before the fused quantizer is launched."""
    assert _w4a4(L, a=NULL) == INVALID
    assert _w4a4(L, M=0) == INVALID
    assert _w4a4(L, K=48) == NOT_SUPPORTED
    assert _w4a4(L, out_dtype=2) == NOT_SUPPORTED
    assert _w4a4(L, n_out=32) == INVALID               # no row_idx: n_out must be N
    assert _w4a4(L, row_idx=P, n_out=65) == INVALID    # more rows than N
    assert _w4a4(L, a=MIS) == INVALID
    assert _w4a4(L, out=MIS) == INVALID
    assert _w4a4(L, row_idx=MIS, n_out=32) == INVALID
    # decode (M=8) quantizes into the workspace; prefill (M=512) too
    for M in (8, 512):
        need = L.nvfp4_gemm_w4a4_bf16_workspace_size(M, 5120, 17408, 5120)
        assert need >= M * 17408 * 2 if M == 8 else need >= M * 17408 // 2 + M * 17408 // 16
        assert _w4a4(L, M=M, N=5120, K=17408, n_out=5120) == WORKSPACE
        assert _w4a4(L, M=M, N=5120, K=17408, n_out=5120, workspace=P, wbytes=need - 1) == WORKSPACE
        assert _w4a4(L, M=M, N=5120, K=17408, n_out=5120, workspace=MIS, wbytes=need) == INVALID
    assert L.nvfp4_gemm_w4a4_bf16_workspace_size(0, 64, 256, 64) == 0

def test_workspace_queries_are_pure(L):
    a = L.nvfp4_gemm_workspace_size(0, 8, 17408, 5120, 17408)
    b = L.nvfp4_gemm_workspace_size(0, 8, 17408, 5120, 17408)
    assert a == b
    assert L.nvfp4_gemm_workspace_size(2, 8, 17408, 5120, 17408) >= a + 8 * 5120 * 2
    assert L.nvfp4_gemm_workspace_size(0, 0, 1, 1, 1) == 0
    assert L.nvfp4_moe_align_workspace_size(4096, 8, 128) >= 128 * 4
    assert L.nvfp4_grouped_gemm_workspace_size(-1, 1, 1, 1) == 0


def test_moe_validation(L):
    ws = L.nvfp4_moe_align_workspace_size(32, 8, 128)
    assert L.nvfp4_moe_align(NULL, NULL, 32, 8, 128, P, P2, P3, NULL, P4, ws, NULL) == INVALID
    assert L.nvfp4_moe_align(P, NULL, 32, 64, 128, P, P2, P3, NULL, P4, ws, NULL) == NOT_SUPPORTED
    assert L.nvfp4_moe_align(P, NULL, 32, 8, 2048, P, P2, P3, NULL, P4, ws, NULL) == NOT_SUPPORTED
    assert L.nvfp4_moe_align(P, P2, 32, 8, 128, P, P2, P3, NULL, P4, ws, NULL) == INVALID
    assert L.nvfp4_moe_align(P, NULL, 32, 8, 128, P, P2, P3, NULL, NULL, 0, NULL) == WORKSPACE
    g = L.nvfp4_grouped_gemm
    assert g(NULL, 32, 256, P, P2, 4, 32, 64, P3, P4, NULL, 0, P, NULL, 0, NULL) == INVALID
    assert g(P, 32, 240, P, P2, 4, 32, 64, P3, P4, NULL, 0, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 32, 256, P, P2, 4, 32, 48, P3, P4, NULL, 1, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 32, 256, P, P2, 4, 32, 64, P3, P4, NULL, 5, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 8, 256, NULL, P2, 4, 32, 64, P3, P4, NULL, 0, P, NULL, 0, NULL) == INVALID
    gs = L.nvfp4_grouped_gemm_scaled  # the same checks, plus a float-aligned scale array
    assert gs(NULL, 32, 256, P, P2, 4, 32, 64, P3, P4, P, NULL, 0, P, NULL, 0, NULL) == INVALID
    assert gs(P, 32, 240, P, P2, 4, 32, 64, P3, P4, P, NULL, 0, P, NULL, 0,
              NULL) == NOT_SUPPORTED
    assert gs(P, 32, 256, P, P2, 4, 32, 64, P3, P4, ctypes.c_void_p(0x10002), NULL, 0, P, NULL,
              0, NULL) == INVALID
    gsp = L.nvfp4_grouped_gemm_scaled_planned
    assert gsp(_plan(gemm_min_m=0), P, 32, 256, P, P2, 4, 32, 64, P3, P4, P, NULL, 0, P, NULL, 0,
               NULL) == INVALID
    c = L.nvfp4_moe_combine
    assert c(P, NULL, 4, 8, 64, P2, NULL) == INVALID
    assert c(P, P2, 4, 8, 60, P3, NULL) == NOT_SUPPORTED
    assert c(P, P2, 0, 8, 64, P3, NULL) == INVALID


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="GPU"):
        nv.quantize(x)


def test_topk_validation(L):
    def tk(logits=P, M=2, n=5000, k=8, ids_map=NULL, values=P2, ids=P3, ws=P4, wbytes=1 << 20):
        return L.nvfp4_topk(logits, M, n, k, ids_map, values, ids, ws, wbytes, NULL)
    assert tk(logits=NULL) == INVALID
    assert tk(k=0) == INVALID
    assert tk(k=5001) == INVALID                       # k > n
    assert tk(n=300, k=257) == NOT_SUPPORTED           # k above 256
    assert tk(M=70000) == NOT_SUPPORTED
    assert tk(values=MIS) == INVALID
    assert L.nvfp4_topk_workspace_size(2, 512, 64) == 0    # one chunk: no workspace
    assert L.nvfp4_topk_workspace_size(2, 2048, 100) == 0
    need = L.nvfp4_topk_workspace_size(2, 5000, 8)
    assert need >= 2 * 3 * 8 * 8
    assert tk(ws=NULL, wbytes=0) == WORKSPACE
    assert tk(wbytes=need - 1) == WORKSPACE


def test_head_topk_validation(L):
    def hk(a=P, M=1, N=1000, K=256, ri=P4, n_out=100, k=4, ws=P, wbytes=1 << 30):
        return L.nvfp4_head_topk(a, M, N, K, P2, P3, ri, n_out, k, P2, P3, ws, wbytes, NULL)
    assert hk(a=NULL) == INVALID
    assert hk(k=101) == INVALID            # k > n_out
    assert hk(k=300, n_out=500) == NOT_SUPPORTED
    assert hk(K=48) == NOT_SUPPORTED
    assert hk(ri=NULL) == INVALID          # no mask: n_out must be N
    assert hk(n_out=1001) == INVALID
    need = L.nvfp4_head_topk_workspace_size(1, 1000, 256, 100, 4)
    assert need >= 100 * 4
    assert hk(ws=NULL, wbytes=0) == WORKSPACE
    assert hk(wbytes=need - 1) == WORKSPACE


def test_kv_codec_validation(L):
    def st(x=P, T=4, W=128, sm=P2, scale=1.0, cache=P3, slots=64):
        return L.nvfp4_kv_store_e4m3(x, T, W, sm, scale, cache, slots, NULL)

    def ld(cache=P, slots=64, W=128, bt=P2, lens=P3, B=2, mp=4, ps=16, ml=64, scale=1.0, out=P4):
        return L.nvfp4_kv_load_e4m3(cache, slots, W, bt, lens, B, mp, ps, ml, scale, out, NULL)
    assert st(x=NULL) == INVALID
    assert st(T=0) == INVALID
    assert st(W=24) == NOT_SUPPORTED
    assert st(scale=0.0) == INVALID
    assert st(scale=float("inf")) == INVALID
    assert st(scale=float("nan")) == INVALID
    assert st(scale=-1.0) == INVALID
    assert st(cache=MIS) == INVALID
    assert ld(bt=NULL) == INVALID
    assert ld(ps=0) == INVALID
    assert ld(W=40) == NOT_SUPPORTED
    assert ld(out=MIS) == INVALID
    assert ld(scale=1e-40) == INVALID


def test_two_level_validation(L):
    G = ctypes.c_void_p(0x50000)
    G_MIS = ctypes.c_void_p(0x50002)
    assert L.nvfp4_quantize_scaled(P, 4, 64, NULL, P2, P3, NULL) == INVALID
    assert L.nvfp4_quantize_scaled(P, 4, 48, G, P2, P3, NULL) == NOT_SUPPORTED
    assert L.nvfp4_quantize_scaled(P, 4, 64, G_MIS, P2, P3, NULL) == INVALID
    need = L.nvfp4_quantize_weight_workspace_size(64, 64)
    assert need > 0
    assert L.nvfp4_quantize_weight(P, 64, 64, P2, P3, G, NULL, 0, NULL) == WORKSPACE
    assert L.nvfp4_quantize_weight(P, 64, 64, P2, P3, G, P4, need - 1, NULL) == WORKSPACE
    assert L.nvfp4_quantize_weight(P, 64, 64, P2, P3, NULL, P4, need, NULL) == INVALID
    assert L.nvfp4_dequantize_scaled(P, P2, NULL, 4, 64, P3, NULL) == INVALID
    assert L.nvfp4_dequantize_scaled(P, P2, G, 4, 40, P3, NULL) == NOT_SUPPORTED

    def gs(a_dtype=0, ag=NULL, wg=G, **kw):
        return L.nvfp4_gemm_scaled(a_dtype, P, P4 if a_dtype == 2 else NULL, ag, 4, 64, 256, P2,
                                   P3, wg, NULL, 64, 0, P4, NULL, 0, NULL)
    assert gs(ag=G) == INVALID                 # activation scale needs NVFP4 activations
    assert gs(wg=G_MIS) == INVALID


def test_mfma_k_limit_is_not_supported(L):
    """The MFMA GEMM's 32-bit activation offsets cap K at 2^22: a longer K at a
    large M is refused on the host (NOT_SUPPORTED), not at launch."""
    K = (1 << 22) + 32
    assert _gemm(L, M=128, N=64, K=K, n_out=64, workspace=P, wbytes=1 << 40) == NOT_SUPPORTED
    assert _w4a4(L, M=128, N=64, K=K, n_out=64, workspace=P, wbytes=1 << 40) == NOT_SUPPORTED


def test_grouped_shape_no_kernel_takes(L):
    """A K past the grouped GEMV's LDS staging runs the MFMA kernel; with 32-bit
    MFMA activation offsets exceeded as well no kernel takes the shape and the
    call returns NOT_SUPPORTED before any launch."""
    g = L.nvfp4_grouped_gemm
    assert g(P, 32768, 65536, NULL, P2, 4, 32768, 64, P3, P4, NULL, 0, P, NULL, 0,
             NULL) == NOT_SUPPORTED


def _plan(**kw):
    return ctypes.byref(nv.make_plan(**kw))


def test_plan_default_is_all_minus_one(L):
    p = nv.Plan()
    L.nvfp4_plan_default(ctypes.byref(p))
    assert all(getattr(p, n) == -1 for n, _ in nv.Plan._fields_)


def test_planned_entry_points_validate_the_plan(L):
    """A plan naming a layout the library does not build is refused with
    INVALID before any HIP call; a default plan behaves as the plain entry
    point (same workspace, same argument checks)."""
    def gp(plan, M=4, **kw):
        return L.nvfp4_gemm_planned(plan, 0, P, NULL, M, 64, 256, P2, P3, NULL, 64, 0, P4, NULL,
                                    0, NULL)
    assert gp(_plan(gemv_tiles=3)) == INVALID            # no 3-tile layout
    assert gp(_plan(gemv_waves=16), M=8) == INVALID       # 16 waves need two activation tiles
    assert gp(_plan(gemv_small_max=9)) == INVALID
    assert gp(_plan(gemv_lds_kib=4)) == INVALID
    assert gp(_plan(gemm_min_m=0)) == INVALID
    assert L.nvfp4_gemm_planned(_plan(), 0, NULL, NULL, 4, 64, 256, P2, P3, NULL, 64, 0, P4,
                                NULL, 0, NULL) == INVALID
    for args in ((0, 8, 17408, 5120, 17408), (0, 32, 5120, 17408, 5120), (2, 512, 17408, 5120,
                                                                          17408)):
        assert (L.nvfp4_gemm_workspace_size_planned(None, *args) ==
                L.nvfp4_gemm_workspace_size(*args))
        assert (L.nvfp4_gemm_workspace_size_planned(_plan(), *args) ==
                L.nvfp4_gemm_workspace_size(*args))
    # the K parts of the plan size the partial workspace
    base = L.nvfp4_gemm_workspace_size(0, 8, 1024, 4096, 1024)
    assert base == 16 * 8 * 1024 * 4
    assert L.nvfp4_gemm_workspace_size_planned(_plan(gemv_splits=2), 0, 8, 1024, 4096,
                                               1024) == 2 * 8 * 1024 * 4
    # the fused W4A4 staging is built for one or two weight tiles per wave
    assert L.nvfp4_gemm_w4a4_bf16_planned(_plan(w4a4_fuse=1, gemv_tiles=4), P, 8, 64, 256, P2, P3,
                                          NULL, 64, 0, P4, NULL, 0, NULL) == INVALID
    assert L.nvfp4_gemm_w4a4_bf16_planned(_plan(w4a4_fuse=2), P, 8, 64, 256, P2, P3, NULL, 64, 0,
                                          P4, NULL, 0, NULL) == INVALID
    # fused W4A4 needs no activation copy in the workspace; the one-pass form does
    fused = L.nvfp4_gemm_w4a4_bf16_workspace_size_planned(_plan(w4a4_fuse=1), 512, 17408, 5120,
                                                          17408)
    pas = L.nvfp4_gemm_w4a4_bf16_workspace_size_planned(_plan(w4a4_fuse=0), 512, 17408, 5120,
                                                        17408)
    assert pas >= fused + 512 * 5120 * 2
    g = L.nvfp4_grouped_gemm_planned
    assert g(_plan(gemm_min_m=0), P, 32, 256, P, P2, 4, 32, 64, P3, P4, NULL, 0, P, NULL, 0,
             NULL) == INVALID
    assert g(_plan(grouped_mfma_min_rows=1), NULL, 32, 256, P, P2, 4, 32, 64, P3, P4, NULL, 0, P,
             NULL, 0, NULL) == INVALID


def test_binding_checks_shapes_before_the_gpu(L):
    """The binding checks every tensor's dtype and exact shape (caller-supplied
    outputs, scales, indices, workspace) before any GPU work: a wrong one is a
    ValueError naming the argument (CPU tensors reach this check first)."""
    import torch
    bf = torch.bfloat16
    u8 = torch.uint8
    x = torch.zeros(4, 256, dtype=bf)
    wc = torch.zeros(64, 128, dtype=u8)
    ws = torch.zeros(64, 16, dtype=u8)

    def raises(match, fn, *a, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k)
    raises("w_scales", nv.gemm, x, wc, torch.zeros(64, 15, dtype=u8))
    raises("K mismatch", nv.gemm, torch.zeros(4, 512, dtype=bf), wc, ws)
    raises("out", nv.gemm, x, wc, ws, out=torch.zeros(4, 64, dtype=bf), out_dtype=torch.float32)
    raises("out", nv.gemm, x, wc, ws, out=torch.zeros(4, 63, dtype=bf))
    raises("row_idx", nv.gemm, x, wc, ws, row_idx=torch.zeros(8, dtype=torch.int64))
    raises("row_idx", nv.gemm, x, wc, ws, row_idx=torch.zeros(65, dtype=torch.int32))
    raises("a_scales", nv.gemm, torch.zeros(4, 128, dtype=u8), wc, ws,
           a_scales=torch.zeros(4, 8, dtype=u8))
    raises("out_dtype", nv.gemm, x, wc, ws, out_dtype=torch.float16)
    raises("codes", nv.quantize, x, codes=torch.zeros(4, 64, dtype=u8))
    raises("x", nv.quantize, torch.zeros(4, 256, dtype=torch.float32))
    raises("out", nv.dequantize, wc, ws, out=torch.zeros(64, 128, dtype=bf))
    raises("global_scale", nv.gemm_scaled, x, wc, ws, w_global_scale=torch.zeros(2))
    raises("out", nv.gemm_w4a4, x, wc, ws, out=torch.zeros(3, 64, dtype=bf))
    w3c = torch.zeros(4, 64, 128, dtype=u8)
    w3s = torch.zeros(4, 64, 16, dtype=u8)
    off = torch.zeros(5, dtype=torch.int32)
    raises("expert_offsets", nv.grouped_gemm, x, None, torch.zeros(4, dtype=torch.int32), w3c,
           w3s, 4)
    raises("row_scale", nv.grouped_gemm, x, None, off, w3c, w3s, 4,
           row_scale=torch.zeros(3, dtype=torch.float32))
    raises("gather_idx", nv.grouped_gemm, x, torch.zeros(4, dtype=torch.int64), off, w3c, w3s, 4)
    raises("out", nv.grouped_gemm, x, None, off, w3c, w3s, 4, epilogue=nv.EPI_SWIGLU,
           out=torch.zeros(4, 64, dtype=bf))
    raises("w_global", nv.grouped_gemm, x, None, off, w3c, w3s, 4,
           w_global=torch.zeros(5, dtype=torch.float32))
    raises("w_global", nv.grouped_gemm, x, None, off, w3c, w3s, 4,
           w_global=torch.zeros(4, dtype=torch.float64))
    raises("rows", nv.moe_combine, torch.zeros(7, 64, dtype=bf), torch.zeros(2, 4, dtype=torch.int32))
    raises("cache", nv.kv_store_e4m3, torch.zeros(4, 64, dtype=bf),
           torch.zeros(4, dtype=torch.int32), 1.0, torch.zeros(8, 32, dtype=u8))
    raises("seq_lens", nv.kv_load_e4m3, torch.zeros(8, 64, dtype=u8),
           torch.zeros(2, 3, dtype=torch.int32), torch.zeros(3, dtype=torch.int32), 16, 48, 1.0)
    raises("ids_map", nv.topk, torch.zeros(2, 100), 4, ids_map=torch.zeros(99, dtype=torch.int32))
    with pytest.raises(RuntimeError, match="GPU"):   # shapes right, tensors on the CPU
        nv.gemm(x, wc, ws)


def test_noalloc_validation(L):
    """nvfp4_gemm_noalloc checks its arguments as nvfp4_gemm does and refuses a
    call that needs more than its device array, all before any HIP call."""
    def na(a_dtype=0, a=P, a_scales=NULL, M=4, N=64, K=256, out=P4, n_out=64):
        return L.nvfp4_gemm_noalloc(a_dtype, a, a_scales, M, N, K, P2, P3, NULL, n_out, 0, out,
                                    NULL)
    assert L.nvfp4_noalloc_scratch_bytes() == 64 << 20
    assert na(a=NULL) == INVALID
    assert na(K=48) == NOT_SUPPORTED
    assert na(a_scales=P) == INVALID
    assert na(a_dtype=2) == INVALID
    assert na(out=MIS) == INVALID
    assert na(n_out=32) == INVALID
    # W4A4 at M = 8192: 80 MiB of dequantized activations alone
    assert na(a_dtype=2, a_scales=P, M=8192, N=256, K=5120, n_out=256) == WORKSPACE


def test_kparts_plan_validation(L):
    """A K-parts plan names a built layout, one activation tile, full 256-element
    steps and at least one step per part; anything else is INVALID before any
    HIP call."""
    def gp(M=8, K=4096, **kw):
        return L.nvfp4_gemm_planned(_plan(**kw), 0, P, NULL, M, 64, K, P2, P3, NULL, 64, 0, P4,
                                    NULL, 0, NULL)
    ok = dict(gemv_tiles=2, gemv_waves=8, gemv_kparts=4)
    assert gp(K=4128, **ok) == INVALID           # K % 256 != 0
    assert gp(K=768, **ok) == INVALID            # 3 steps, 4 parts
    assert gp(M=3, **ok) == INVALID              # the 4x4x4-block GEMV takes M <= 4
    assert gp(M=20, **ok) == INVALID             # two activation tiles
    assert gp(gemv_tiles=2, gemv_waves=16, gemv_kparts=4) == INVALID   # no (2, 16, 4)
    assert gp(M=12, gemv_tiles=2, gemv_waves=16, gemv_kparts=8) == INVALID  # 8 parts need M <= 8
    assert (L.nvfp4_gemm_workspace_size_planned(_plan(**ok), 0, 8, 64, 4096, 64) == 0)


def test_tiled_validation(L):
    """nvfp4_tiled_weight_bytes, nvfp4_tile_weight and nvfp4_gemm_tiled reject
    bad arguments on the host."""
    assert L.nvfp4_tiled_weight_bytes(17, 288) == 2 * 2 * 2304
    assert L.nvfp4_tiled_weight_bytes(248320, 5120) == 248320 * 5120 * 9 // 16
    assert L.nvfp4_tiled_weight_bytes(16, 48) == 0  # K % 32 != 0
    assert L.nvfp4_tiled_weight_bytes(0, 64) == 0
    t = L.nvfp4_tile_weight  # (codes, scales, N, K, row_idx, n_rows, w_tiled, stream)
    assert t(NULL, P2, 4, 64, NULL, 4, P3, NULL) == INVALID
    assert t(P, P2, 4, 64, NULL, 4, NULL, NULL) == INVALID
    assert t(P, P2, 0, 64, NULL, 0, P3, NULL) == INVALID
    assert t(P, P2, 4, 48, NULL, 4, P3, NULL) == NOT_SUPPORTED
    assert t(MIS, P2, 4, 64, NULL, 4, P3, NULL) == INVALID
    assert t(P, P2, 4, 64, NULL, 3, P3, NULL) == INVALID  # all rows: n_rows == N
    assert t(P, P2, 4, 64, P4, 5, P3, NULL) == INVALID    # a subset: n_rows <= N
    assert t(P, P2, 4, 64, P4, 0, P3, NULL) == INVALID
    assert t(P, P2, 4, 64, MIS, 2, P3, NULL) == INVALID
    # more 16-byte pieces than one launch of 256-thread workgroups covers
    assert t(P, P2, 1 << 30, 32768, NULL, 1 << 30, P3, NULL) == NOT_SUPPORTED
    g = L.nvfp4_gemm_tiled
    # (a_dtype, a, a_scales, M, N, K, w_tiled, out_dtype, out, ws, ws_bytes, stream)
    assert g(0, NULL, NULL, 1, 16, 64, P2, 0, P3, NULL, 0, NULL) == INVALID
    assert g(0, P, NULL, 1, 16, 64, NULL, 0, P3, NULL, 0, NULL) == INVALID
    assert g(0, P, NULL, 0, 16, 64, P2, 0, P3, NULL, 0, NULL) == INVALID
    assert g(0, P, NULL, 1, 16, 48, P2, 0, P3, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(0, P, NULL, 1, 16, 64, P2, 7, P3, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(5, P, NULL, 1, 16, 64, P2, 0, P3, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(0, P, NULL, 1, 16, 64, MIS, 0, P3, NULL, 0, NULL) == INVALID
    assert g(0, P, P4, 1, 16, 64, P2, 0, P3, NULL, 0, NULL) == INVALID  # bf16 with scales
    assert g(2, P, NULL, 1, 16, 64, P2, 0, P3, NULL, 0, NULL) == INVALID  # NVFP4 without
    need = L.nvfp4_gemm_tiled_workspace_size(0, 8, 17408, 5120)
    assert need > 0
    assert g(0, P, NULL, 8, 17408, 5120, P2, 0, P3, NULL, 0, NULL) == WORKSPACE
    assert g(0, P, NULL, 8, 17408, 5120, P2, 0, P3, P4, need - 1, NULL) == WORKSPACE
    # W4A4 needs room for the dequantized activations
    assert L.nvfp4_gemm_tiled_workspace_size(2, 8, 17408, 5120) >= need + 8 * 5120 * 2


def test_tiled_plan_validation(L):
    """Tiled plans that name no built layout are refused before any launch."""
    def planned(**f):
        p = nv.make_plan(**f)
        return L.nvfp4_gemm_tiled_planned(ctypes.byref(p), 0, P, NULL, 8, 1024, 2048, P2, 0, P3,
                                          P4, 1 << 30, NULL)
    assert planned(gemv_kparts=2) == INVALID
    assert planned(gemv_small_max=9) == INVALID
    assert planned(gemv_tiles=3) == INVALID
    assert planned(gemv_waves=16) == INVALID  # 16 waves need two activation tiles
    assert planned(gemv_small_max=8, gemv_tiles=4) == INVALID
    assert planned(gemv_lds_kib=4) == INVALID


def test_grouped_tiled_validation(L):
    """nvfp4_grouped_gemm_tiled: the grouped checks with the tiled weights in
    place of the codes/scales pair (no scales pointer); the planned variant
    refuses a grouped GEMV wave count that is not built."""
    g = L.nvfp4_grouped_gemm_tiled
    # (a, a_rows, K, gather, offsets, E, R, N, w_tiled, w_global, row_scale, epi, out, ws, wsb, st)
    assert g(NULL, 32, 256, P, P2, 4, 32, 64, P3, NULL, NULL, 0, P, NULL, 0, NULL) == INVALID
    assert g(P, 32, 256, P, P2, 4, 32, 64, NULL, NULL, NULL, 0, P, NULL, 0, NULL) == INVALID
    assert g(P, 32, 240, P, P2, 4, 32, 64, P3, NULL, NULL, 0, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 32, 256, P, P2, 4, 32, 48, P3, NULL, NULL, 1, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 32, 256, P, P2, 4, 32, 56, P3, NULL, NULL, 0, P, NULL, 0, NULL) == NOT_SUPPORTED
    assert g(P, 32, 256, P, P2, 4, 32, 64, MIS, NULL, NULL, 0, P, NULL, 0, NULL) == INVALID
    assert g(P, 32, 256, P, P2, 4, 32, 64, P3, ctypes.c_void_p(0x10002), NULL, 0, P, NULL, 0,
             NULL) == INVALID
    gp = L.nvfp4_grouped_gemm_tiled_planned
    for waves in (3, 12, 32):
        p = nv.make_plan(grouped_gemv_waves=waves)
        assert gp(ctypes.byref(p), P, 32, 256, P, P2, 4, 32, 64, P3, NULL, NULL, 0, P, NULL, 0,
                  NULL) == INVALID


def test_binding_checks_tiled_shapes(L):
    """The tiled binding functions check sizes and dtypes before any GPU work."""
    import torch
    bf, u8 = torch.bfloat16, torch.uint8
    x = torch.zeros(4, 256, dtype=bf)
    wc = torch.zeros(64, 128, dtype=u8)
    ws = torch.zeros(64, 16, dtype=u8)
    nb = nv.tiled_weight_bytes(64, 256)
    assert nb == 4 * 1 * 2304

    def raises(match, fn, *a, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k)
    raises("w_scales", nv.tile_weight, wc, torch.zeros(64, 15, dtype=u8))
    raises("out", nv.tile_weight, wc, ws, out=torch.zeros(nb - 1, dtype=u8))
    raises("row_idx", nv.tile_weight, wc, ws, row_idx=torch.zeros(65, dtype=torch.int32))
    raises("w_tiled", nv.gemm_tiled, x, torch.zeros(nb + 16, dtype=u8), 64)
    raises("w_tiled", nv.gemm_tiled, x, torch.zeros(nb, dtype=u8), 65)
    raises("out", nv.gemm_tiled, x, torch.zeros(nb, dtype=u8), 64,
           out=torch.zeros(4, 64, dtype=bf), out_dtype=torch.float32)
    raises("multiple of 16", nv.tile_experts, torch.zeros(2, 24, 128, dtype=u8),
           torch.zeros(2, 24, 16, dtype=u8))
    off = torch.zeros(3, dtype=torch.int32)
    raises("w_tiled", nv.grouped_gemm_tiled, x, None, off, torch.zeros(nb, dtype=u8), 2, 64, 4)
    raises("expert_offsets", nv.grouped_gemm_tiled, x, None, torch.zeros(2, dtype=torch.int32),
           torch.zeros(nv.tiled_weight_bytes(128, 256), dtype=u8), 2, 64, 4)
