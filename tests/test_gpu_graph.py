"""nvfp4_gemm calls captured in a HIP graph: every replay (with eager work and
synchronisations between replays) must reproduce the eager results bit for
bit -- the benchmark replays its decode step this way.  Covers a split-K GEMV
with workspace, the 4x4x4 small-M kernel, a masked-row call and the MFMA GEMM,
and the other entry points the benchmark replays."""
import numpy as np
import pytest

import helpers
import workloads

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import bit_quantized_gemm_nvfp4_amd as nv
    helpers.announce("graph capture of nvfp4_gemm calls")
    rng = np.random.default_rng(60)
    K, N = 2048, 1536
    w = workloads.nvfp4_weight(rng, N, K)
    wc, ws = helpers.dev_u8(w.codes), helpers.dev_u8(w.scales)
    idx = helpers.dev_i32(np.sort(rng.choice(N, 300, replace=False)).astype(np.int32))
    cases = []
    for M, ri in [(1, None), (8, None), (32, idx), (300, None)]:
        x = helpers.dev_bf16(workloads.normal_bf16(rng, M, K))
        n_out = N if ri is None else ri.numel()
        out = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")
        wsb = nv.gemm_workspace_size(M, N, K, n_out)
        wsp = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        cases.append((x, ri, out, wsp))

    def run_all():
        for x, ri, out, wsp in cases:
            nv.gemm(x, wc, ws, row_idx=ri, out=out, workspace=wsp)

    run_all()
    torch.cuda.synchronize()
    eager = [c[2].clone() for c in cases]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run_all()
    for rep in range(3):
        for c in cases:
            c[2].fill_(0)
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, out, _), ref in zip(cases, eager):
            assert torch.equal(out, ref), f"replay {rep} differs"
        del junk


def test_graph_replays_other_entry_points():
    """The other calls the benchmark replays from HIP graphs -- the routed MoE
    layer (align, two grouped GEMMs, combine) at a decode and a prefill size,
    the masked-head draft proposal, the quantizer, the fused W4A4 entry, the
    offline weight quantizer and the FP8 KV store and load -- captured once and
    replayed three times with eager work and synchronisations between replays;
    every replay reproduces the eager outputs bit for bit."""
    import torch
    import bit_quantized_gemm_nvfp4_amd as nv
    helpers.announce("graph capture of the MoE layer, head top-k, quantizers, KV codec")
    rng = np.random.default_rng(61)
    moes = []
    for T in (24, 1024):
        wl = workloads.moe(T, E=16, topk=4, H=512, I=256, seed=T)
        moes.append((helpers.dev_bf16(wl.x), helpers.dev_i32(wl.ids), helpers.dev_f32(wl.gates),
                     helpers.dev_u8(wl.w1.codes), helpers.dev_u8(wl.w1.scales),
                     helpers.dev_u8(wl.w2.codes), helpers.dev_u8(wl.w2.scales)))
    K, N = 1024, 4096
    head = workloads.nvfp4_weight(rng, N, K)
    hc, hs = helpers.dev_u8(head.codes), helpers.dev_u8(head.scales)
    hidx = helpers.dev_i32(np.sort(rng.choice(N, 1000, replace=False)).astype(np.int32))
    xh = helpers.dev_bf16(workloads.normal_bf16(rng, 8, K))
    xq = helpers.dev_bf16(workloads.normal_bf16(rng, 64, K, outlier_frac=0.01))
    wq = helpers.dev_bf16(workloads.normal_bf16(rng, 256, K))
    st = workloads.kv_store(300, W=256, seed=3)
    x_kv, slots_kv = helpers.dev_bf16(st.x), helpers.dev_i32(st.slot_mapping)
    cache0 = torch.zeros((st.num_slots, 256), dtype=torch.uint8, device="cuda")
    cache_ld, bt, lens, sc_ld = workloads.kv_load(4, 200, W=256, seed=4)
    cache_ld, bt, lens = helpers.dev_u8(cache_ld), helpers.dev_i32(bt), helpers.dev_i32(lens)

    def run_all():
        outs = [nv.moe_layer(*m) for m in moes]
        outs += list(nv.head_topk(xh, hc, hs, 8, row_idx=hidx))
        outs += list(nv.quantize(xq))
        outs.append(nv.gemm_w4a4(xq, hc, hs))
        outs += list(nv.quantize_weight(wq))
        cache = cache0.clone()
        nv.kv_store_e4m3(x_kv, slots_kv, st.scale, cache)
        outs.append(cache)
        outs.append(nv.kv_load_e4m3(cache_ld, bt, lens, 16, 200, sc_ld))
        return outs

    eager = [o.clone() for o in run_all()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        captured = run_all()
    for rep in range(3):
        for o in captured:
            o.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(captured, eager)):
            assert torch.equal(o, ref), f"replay {rep}: output {i} differs"
        del junk
