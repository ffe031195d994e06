"""nvfp4_gemm calls captured in a HIP graph: every replay (with eager work and
synchronisations between replays) must reproduce the eager results bit for
bit -- the benchmark replays its decode step this way.  Covers a split-K GEMV
with workspace, the 4x4x4 small-M kernel, a masked-row call and the MFMA GEMM."""
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
