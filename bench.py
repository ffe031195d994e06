#!/usr/bin/env python3
"""Benchmark of the NVFP4 linear layer on one MI355X.

Workload of the headline metric (weight-stream GB/s at M = 1..32): the
decode-shaped W4A16 set -- M in {1, 8, 32} x (K, N) in {(5120, 17408),
(17408, 5120), (5120, 248320)} plus the masked head (32,768 of the 248,320
rows) -- 12 calls.  The weights are tiled once before timing
(nvfp4_tile_weight: the same bytes in the streaming kernels' order, as a serving
engine lays out its weights at load; the masked head's fixed id set of 32,768
rows as a matrix of its own) and every call runs nvfp4_gemm_tiled.  One step runs all 12 calls once; `value` is the weight bytes the
step streams (rows * K * 9/16 per call) divided by the step time, with every
input resident in HBM before the timed region starts.  The step is captured
once as a HIP graph and replayed (as a serving engine replays its decode
step); the same calls launched one by one give config.eager_GBs and the
per-call event times of the roofline.  config.row_major repeats the step with
every call on the row-major layout (nvfp4_gemm; the masked head gathering its
rows per call through row_idx).

Infinity-cache (MALL, 256 MB) hygiene: dense weights exist in two copies that
calls alternate, and the head in three: the full-head calls alternate copies 0
and 1, and the masked-head calls read copy 2, which no full-head call reads.
Between two reads of one copy the step streams at least one other full head
(715 MB, far more than the cache), so no call re-reads weights still cached.

Also reported on the same JSON line:
  roofline      -- the decode GEMV kernel: algorithmic weight bytes per launch
                   over its mean launch time (HIP events on the launch stream),
                   against the 8 TB/s HBM peak; `traffic` is the HBM bytes per
                   step measured with the FETCH_SIZE / WRITE_SIZE counters
                   (profiles/decode_gemv_set_hbm_traffic.md), null once the
                   kernel sources differ from the ones measured;
  cpu_baseline  -- the CPU oracle timed on this host on a bounded sample of the
                   same workload (a subset of output rows), scaled to GB/s;
  secondary     -- the other rows of the layer, each graph-replayed (prefill GEMM TFLOP/s,
                   quantizer GB/s, W4A4 GEMM TFLOP/s, FP8 KV-cache store/load
                   GB/s, MoE layer T=32 / T=4096); prefill and MoE also on tiled
                   weights (*_tiled_* rows);
  draft_proposal -- the masked head with its top-8 proposal (nvfp4_head_topk)
                   against the head GEMV alone, graph-replayed, M in {1, 8, 32}.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
COPY_PROBE_BYTES = 256 << 20
METRIC = "NVFP4 GEMM: weight-stream GB/s at M=1..32; TFLOP/s at M=8192 (1 GPU)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_gemv_set_hbm_traffic.md")


def measured_traffic():
    """HBM bytes per decode step from the committed FETCH_SIZE / WRITE_SIZE
    counter summary, or None when the GEMV kernel sources have changed since
    the counters were taken (their SHA-256 is recorded beside the figure)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        k, sep, v = line.partition(":")
        if sep and k.strip() in ("traffic_bytes_per_step", "kernel_sources_sha256", "kernel_sources"):
            fields[k.strip()] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for name in fields["kernel_sources"].split():
        path = os.path.join(ROOT, "bit_quantized_gemm_nvfp4_amd", "csrc", name)
        try:
            h.update(open(path, "rb").read())
        except OSError:
            return None
    if h.hexdigest() != fields["kernel_sources_sha256"]:
        return None
    return int(fields["traffic_bytes_per_step"])


def weight_bytes(rows: int, K: int) -> int:
    return rows * K * 9 // 16


class Decode:
    """The 12-call decode set with its weight copies, all resident on the GPU.

    With tiled=True (the serving configuration) every call reads weights in the
    tiled layout (nvfp4_tile_weight, done once here, as an engine does when it
    loads the weights) through nvfp4_gemm_tiled: the nine dense calls their
    whole matrices, the masked head the 32,768 rows of its fixed id set, tiled
    as a matrix of their own.  With tiled=False every call reads the row-major
    layout through nvfp4_gemm, the masked head gathering its rows per call
    (row_idx)."""

    def __init__(self, nv, torch, helpers_dev, tiled=True):
        import workloads as wl
        self.nv, self.torch = nv, torch
        dev_u8, dev_bf16, dev_i32 = helpers_dev
        self.calls = []  # (name, M, K, rows, fn)
        shapes = wl.DECODE_SHAPES
        self.weights = {}
        for (K, N) in shapes:
            w = wl.decode_weights(K, N)
            copies = [(dev_u8(w.codes), dev_u8(w.scales))]
            n_copies = 3 if (K, N) == (wl.HIDDEN, wl.VOCAB) else 2
            for _ in range(n_copies - 1):
                copies.append((copies[0][0].clone(), copies[0][1].clone()))
            self.weights[(K, N)] = copies
            del w
        self.idx = dev_i32(wl.decode_masked_rows())
        self.x = {(M, K): dev_bf16(wl.decode_activations(M, K))
                  for M in wl.DECODE_M for K in {s[0] for s in shapes}}
        self.keep = []
        self.tiled = tiled
        if tiled:  # the dense calls' copies 0 and 1 in the tiled layout, and the
            # masked head's rows (its id set is fixed) tiled from head copy 2
            self.tiled_weights = {s: [nv.tile_weight(*self.weights[s][c]) for c in range(2)]
                                  for s in shapes}
            self.tiled_masked = nv.tile_weight(*self.weights[(wl.HIDDEN, wl.VOCAB)][2],
                                               row_idx=self.idx)
        head = (wl.HIDDEN, wl.VOCAB)
        call_no = 0
        for M in wl.DECODE_M:
            for (K, N) in shapes:
                c = call_no % 2
                if tiled:
                    self._add_tiled(f"M{M}_K{K}_N{N}", M, K, N, self.tiled_weights[(K, N)][c])
                else:
                    self._add(f"M{M}_K{K}_N{N}", M, K, N, self.weights[(K, N)][c], None, N)
                call_no += 1
            # masked head: its own copy, which no full-head call reads
            K, N = head
            if tiled:
                self._add_tiled(f"M{M}_masked_head", M, K, self.idx.numel(), self.tiled_masked)
            else:
                self._add(f"M{M}_masked_head", M, K, N, self.weights[head][2], self.idx,
                          self.idx.numel())
        torch.cuda.synchronize()

    def _add(self, name, M, K, N, w, idx, n_out):
        """One nvfp4_gemm call with its arguments marshalled once: the timed loop
        calls the C entry point directly on torch's current stream."""
        import ctypes
        torch, nv = self.torch, self.nv
        out = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")
        wsb = nv.gemm_workspace_size(M, N, K, n_out)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
        x = self.x[(M, K)]
        wc, wsc = w
        self.keep.append((out, ws))
        vp = ctypes.c_void_p
        args = (nv.BF16, vp(x.data_ptr()), None, M, N, K, vp(wc.data_ptr()), vp(wsc.data_ptr()),
                None if idx is None else vp(idx.data_ptr()), n_out, nv.BF16, vp(out.data_ptr()),
                None if ws is None else vp(ws.data_ptr()), wsb)
        f = nv.lib().nvfp4_gemm

        def fn(stream=None, f=f, args=args):
            st = torch.cuda.current_stream().cuda_stream if stream is None else stream
            rc = f(*args, vp(st))
            if rc != 0:
                raise RuntimeError(nv.lib().nvfp4_status_string(rc).decode())

        self.calls.append((name, M, K, n_out, fn))

    def _add_tiled(self, name, M, K, N, wt):
        """One nvfp4_gemm_tiled call, arguments marshalled once."""
        import ctypes
        torch, nv = self.torch, self.nv
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        wsb = nv.gemm_tiled_workspace_size(M, N, K)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
        x = self.x[(M, K)]
        self.keep.append((out, ws))
        vp = ctypes.c_void_p
        args = (nv.BF16, vp(x.data_ptr()), None, M, N, K, vp(wt.data_ptr()), nv.BF16,
                vp(out.data_ptr()), None if ws is None else vp(ws.data_ptr()), wsb)
        f = nv.lib().nvfp4_gemm_tiled

        def fn(stream=None, f=f, args=args):
            st = torch.cuda.current_stream().cuda_stream if stream is None else stream
            rc = f(*args, vp(st))
            if rc != 0:
                raise RuntimeError(nv.lib().nvfp4_status_string(rc).decode())

        self.calls.append((name, M, K, N, fn))

    def step_bytes(self):
        return sum(weight_bytes(rows, K) for (_, _, K, rows, _) in self.calls)


def time_decode_graph(dec, torch, steps, warmup):
    """The step captured once as a HIP graph (how a serving engine replays a
    decode step) and replayed: returns the wall time of `steps` replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in dec.calls:
            c[4](side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for c in dec.calls:
            c[4](side.cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # the GPU idled while the graph was captured: replay it (untimed) for
    # ~0.2 s more, so the timed replays see the clocks settled under load again
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_decode(dec, torch, steps, warmup):
    """Per-call pass: every call launched on its own, bracketed by HIP events on
    the launch stream.  Warm-up and timed calls are enqueued without a
    synchronisation between them, so the host runs ahead of the GPU and each
    event pair brackets one kernel (plus its split-K reduce) running back to
    back with the others, not the host's launch gaps."""
    n = len(dec.calls)
    starts = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
    ends = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
    torch.cuda.synchronize()
    for _ in range(warmup):
        for c in dec.calls:
            c[4]()
    for s in range(steps):
        for i, c in enumerate(dec.calls):
            starts[s][i].record()
            c[4]()
            ends[s][i].record()
    torch.cuda.synchronize()
    wall = starts[0][0].elapsed_time(ends[-1][-1]) / 1e3
    per_call_ms = np.array([[starts[s][i].elapsed_time(ends[s][i]) for i in range(n)]
                            for s in range(steps)])
    return wall, per_call_ms


def time_draft(dec, torch, nv, k=8, reps=20, replays=5):
    """Draft proposal of the masked head (nvfp4_head_topk: head GEMV over the
    32,768 kept rows, then the top-k) against the head GEMV alone, each call
    captured `reps` times in a HIP graph and replayed, for M in {1, 8, 32}."""
    import ctypes
    import workloads as wl
    K, N = wl.HIDDEN, wl.VOCAB
    wc, wsc = dec.weights[(K, N)][0]
    idx = dec.idx
    n_out = idx.numel()
    vp = ctypes.c_void_p
    L = nv.lib()
    res = {}

    def graph_us(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(side.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(reps):
                fn(side.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (replays * reps) * 1e6

    for M in wl.DECODE_M:
        x = dec.x[(M, K)]
        vals = torch.empty((M, k), dtype=torch.float32, device="cuda")
        ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
        logits = torch.empty((M, n_out), dtype=torch.float32, device="cuda")
        wsb = max(nv.head_topk_workspace_size(M, N, K, n_out, k),
                  nv.gemm_workspace_size(M, N, K, n_out))
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

        def head(st):
            rc = L.nvfp4_head_topk(vp(x.data_ptr()), M, N, K, vp(wc.data_ptr()),
                                   vp(wsc.data_ptr()), vp(idx.data_ptr()), n_out, k,
                                   vp(vals.data_ptr()), vp(ids.data_ptr()), vp(ws.data_ptr()),
                                   wsb, vp(st))
            assert rc == 0, rc

        def gemv(st):
            rc = L.nvfp4_gemm(nv.BF16, vp(x.data_ptr()), None, M, N, K, vp(wc.data_ptr()),
                              vp(wsc.data_ptr()), vp(idx.data_ptr()), n_out, nv.FP32,
                              vp(logits.data_ptr()), vp(ws.data_ptr()), wsb, vp(st))
            assert rc == 0, rc

        th, tg = graph_us(head), graph_us(gemv)
        res[f"M{M}_head_topk{k}_us"] = round(th, 2)
        res[f"M{M}_head_gemv_us"] = round(tg, 2)
        res[f"M{M}_head_topk{k}_weight_GBs"] = round(weight_bytes(n_out, K) / (th * 1e-6) / 1e9, 1)
    return res


def cpu_baseline(target_s=15.0):
    """The oracle on this host, on a bounded sample of the same workload: every
    call of the decode step restricted to an evenly spaced subset of its output
    rows (same activations, same weight rows), scaled to weight-stream GB/s.
    A 1/512-row pass calibrates the subset so the timed pass takes ~target_s."""
    import oracle
    import workloads as wl
    calls = []  # (M, K, x, codes, scales) with all rows the step reads
    for M in wl.DECODE_M:
        for (K, N) in wl.DECODE_SHAPES:
            calls.append((M, K, N, None))
        calls.append((M, wl.HIDDEN, wl.VOCAB, wl.decode_masked_rows()))
    weights = {s: wl.decode_weights(*s) for s in wl.DECODE_SHAPES}
    xs = {(M, K): wl.decode_activations(M, K) for M in wl.DECODE_M for K in (wl.HIDDEN, wl.MLP)}

    def run(frac):
        t, b = 0.0, 0
        for (M, K, N, idx) in calls:
            rows = np.arange(N) if idx is None else idx
            n = max(1, int(len(rows) * frac))
            sel = rows[np.linspace(0, len(rows) - 1, n).astype(np.int64)]
            w = weights[(K, N)]
            wc, ws = w.codes[sel], w.scales[sel]
            t0 = time.perf_counter()
            oracle.gemm_w4a16(xs[(M, K)], M, K, wc, ws)
            t += time.perf_counter() - t0
            b += weight_bytes(n, K)
        return t, b

    t1, _ = run(1 / 512)
    frac = min(1.0, (1 / 512) * target_s / max(t1, 1e-3))
    t, b = run(frac)
    return {
        "value": round(b / t / 1e9, 5),
        "unit": "GB/s",
        "cores": int(oracle.num_threads()),
        "kind": "oracle",
        "sample": (f"all 12 decode calls, each on {frac:.4%} of its output rows (evenly spaced): "
                   f"{b} weight bytes in {t:.2f} s"),
    }


def _graph_timer(torch):
    def timeit(fn, n=3, warm_s=0.03, timed_s=0.03):
        """Seconds per call: n calls captured in one HIP graph (so the host-side
        cost of the binding is not measured), replayed for ~warm_s of GPU time
        (the clocks settle under sustained load: a lone first call of the
        prefill GEMM runs ~15% slower), then timed over >= 2 replays and
        ~timed_s."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        t_replay = max(a.elapsed_time(b) / 1e3, 1e-6)
        for _ in range(int(warm_s / t_replay)):
            g.replay()
        reps_t = max(2, int(timed_s / t_replay))
        a.record()
        for _ in range(reps_t):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (reps_t * n) / 1e3
    return timeit


def _row(value, unit, peak):
    """A secondary row: the figure, its unit and its fraction of the MI355X
    peak that bounds it (HBM 8 TB/s, or dense bf16 MFMA 2.5 PFLOP/s)."""
    return {"value": round(value, 2), "unit": unit, "frac": round(value / peak, 4)}


def _tf(flop, t):
    return _row(flop / t / 1e12, "TFLOP/s", BF16_MFMA_PEAK_TFLOPS)


def _gb(nbytes, t):
    return _row(nbytes / t / 1e9, "GB/s", HBM_PEAK_GBS)


SECONDARY_CASES = ["prefill_K5120", "prefill_K17408", "quantize", "w4a4", "w4a4_decode",
                   "quantize_weight", "kv", "moe_T32", "moe_T4096"]


def secondary(nv, torch, helpers_dev, cases=None):
    """Single-GPU timings of the other rows of the layer, graph-replayed; each
    with its roofline fraction.  `cases` selects a subset (profiling)."""
    import workloads as wl
    dev_u8, dev_bf16, dev_i32 = helpers_dev
    timeit = _graph_timer(torch)
    res = {}
    cases = SECONDARY_CASES if cases is None else cases

    def prefill(K, N):
        log(f"secondary: prefill K={K} N={N}")
        x, w = wl.prefill(K, N)
        xd, wc, ws = dev_bf16(x), dev_u8(w.codes), dev_u8(w.scales)
        del x, w
        out = torch.empty((8192, N), dtype=torch.bfloat16, device="cuda")
        wsz = nv.gemm_workspace_size(8192, N, K, N)
        wsb = torch.empty(max(wsz, 1), dtype=torch.uint8, device="cuda")
        t = timeit(lambda: nv.gemm(xd, wc, ws, out=out, workspace=wsb), n=1)
        res[f"prefill_M8192_K{K}_N{N}"] = _tf(2 * 8192 * N * K, t)
        # the same product on weights tiled once (nvfp4_gemm_tiled: MFMA GEMM)
        wt = nv.tile_weight(wc, ws)
        wszt = nv.gemm_tiled_workspace_size(8192, N, K)
        wsbt = torch.empty(max(wszt, 1), dtype=torch.uint8, device="cuda")
        t = timeit(lambda: nv.gemm_tiled(xd, wt, N, out=out, workspace=wsbt), n=1)
        res[f"prefill_tiled_M8192_K{K}_N{N}"] = _tf(2 * 8192 * N * K, t)

    if "prefill_K5120" in cases:
        prefill(wl.HIDDEN, wl.MLP)
    if "prefill_K17408" in cases:
        prefill(wl.MLP, wl.HIDDEN)
    if "quantize" in cases:
        log("secondary: quantize")
        for M in (512, 8192):
            xq = dev_bf16(wl.normal_bf16(np.random.default_rng(0), M, wl.HIDDEN, 0.001))
            t = timeit(lambda: nv.quantize(xq), n=20)
            res[f"quantize_M{M}_K5120"] = _gb(M * wl.HIDDEN * (2 + 9 / 16), t)
    if "w4a4" in cases:
        # W4A4 from NVFP4 codes (dequantize pass + bf16 MFMA GEMM), and from bf16
        # activations with the quantizer fused into the MFMA tile loads (fuse=1)
        # or in one pass before the bf16-activation GEMM (fuse=0, the default)
        log("secondary: W4A4")
        _, w = wl.w4a4()
        wc, ws = dev_u8(w.codes), dev_u8(w.scales)
        for M in (512, 8192):
            x = wl.normal_bf16(np.random.default_rng(0), M, wl.HIDDEN, 0.001)
            xd = dev_bf16(x)
            codes, scales = nv.quantize(xd)
            out = torch.empty((M, wl.MLP), dtype=torch.bfloat16, device="cuda")
            fl = 2 * M * wl.MLP * wl.HIDDEN
            n = 3 if M == 512 else 1
            t = timeit(lambda: nv.gemm(codes, wc, ws, a_scales=scales, out=out), n=n)
            res[f"w4a4_codes_M{M}_N17408_K5120"] = _tf(fl, t)
            for fuse in (0, 1):
                pl = {"w4a4_fuse": fuse}
                wsb = torch.empty(max(1, int(nv.lib().nvfp4_gemm_w4a4_bf16_workspace_size_planned(
                    nv._plan_ref(pl), M, wl.MLP, wl.HIDDEN, wl.MLP))), dtype=torch.uint8,
                    device="cuda")
                t = timeit(lambda: nv.gemm_w4a4(xd, wc, ws, out=out, workspace=wsb, plan=pl), n=n)
                res[f"w4a4_bf16_fuse{fuse}_M{M}_N17408_K5120"] = _tf(fl, t)
            del xd, codes, scales, out
    if "w4a4_decode" in cases:
        log("secondary: W4A4 decode shapes")
        _, w = wl.w4a4()
        wc, ws = dev_u8(w.codes), dev_u8(w.scales)
        wb = wl.MLP * wl.HIDDEN * 9 / 16
        for M in (1, 8, 32):
            xm = dev_bf16(wl.normal_bf16(np.random.default_rng(M), M, wl.HIDDEN, 0.001))
            om = torch.empty((M, wl.MLP), dtype=torch.bfloat16, device="cuda")
            t_f = timeit(lambda: nv.gemm_w4a4(xm, wc, ws, out=om), n=20)

            def unfused():
                ac, as_ = nv.quantize(xm)
                nv.gemm(ac, wc, ws, a_scales=as_, out=om)
            t_u = timeit(unfused, n=20)
            res[f"w4a4_fused_M{M}_K5120_N17408"] = dict(_gb(wb, t_f), us=round(t_f * 1e6, 2))
            res[f"w4a4_quantize_then_gemm_M{M}_K5120_N17408"] = dict(_gb(wb, t_u),
                                                                    us=round(t_u * 1e6, 2))
    if "quantize_weight" in cases:
        log("secondary: offline weight quantizer")
        wq = dev_bf16(wl.normal_bf16(np.random.default_rng(1), wl.MLP, wl.HIDDEN))
        wqs = torch.empty(nv.lib().nvfp4_quantize_weight_workspace_size(wl.MLP, wl.HIDDEN),
                          dtype=torch.uint8, device="cuda")
        t = timeit(lambda: nv.quantize_weight(wq, workspace=wqs), n=10)
        # two reads of the bf16 weights (amax pass, quantize pass), codes + scales out
        res["quantize_weight_N17408_K5120"] = _gb(wl.MLP * wl.HIDDEN * (2 + 2 + 9 / 16), t)
        del wq, wqs
    if "kv" in cases:
        log("secondary: KV cache store / load")
        kw = wl.kv_store(8192)
        kx, ksm = dev_bf16(kw.x), dev_i32(kw.slot_mapping)
        kc = torch.zeros((kw.num_slots, wl.KV_W), dtype=torch.uint8, device="cuda")
        t = timeit(lambda: nv.kv_store_e4m3(kx, ksm, kw.scale, kc), n=20)
        res["kv_store_T8192_W1024"] = _gb(8192 * wl.KV_W * 3, t)
        cache, bt, lens, kscale = wl.kv_load(32, 4096)
        kc2, kbt, kl = dev_u8(cache), dev_i32(bt), dev_i32(lens)
        kout = torch.empty((32, 4096, wl.KV_W), dtype=torch.bfloat16, device="cuda")
        t = timeit(lambda: nv.kv_load_e4m3(kc2, kbt, kl, wl.KV_PAGE, 4096, kscale, out=kout),
                   n=10)
        used = int(lens.sum()) * wl.KV_W
        res["kv_load_B32_L4096_W1024"] = _gb(used * 3 + (32 * 4096 * wl.KV_W - used) * 2, t)
        del kx, ksm, kc, kc2, kbt, kl, kout, cache
    for T in (32, 4096):
        if f"moe_T{T}" not in cases:
            continue
        log(f"secondary: MoE T={T}")
        m = wl.moe(T)
        E, topk = 128, 8
        R = T * topk
        x, ids = dev_bf16(m.x), dev_i32(m.ids)
        gates = torch.from_numpy(m.gates).cuda()
        w1c, w1s = dev_u8(m.w1.codes), dev_u8(m.w1.scales)
        w2c, w2s = dev_u8(m.w2.codes), dev_u8(m.w2.scales)
        t = timeit(lambda: nv.moe_layer(x, ids, gates, w1c, w1s, w2c, w2s))
        touched = len(np.unique(m.ids))
        flop = 2 * R * (1536 * 2048 + 2048 * 768)
        wbytes = touched * (1536 * 2048 + 2048 * 768) * 9 // 16
        res[f"moe_T{T}_layer"] = dict(_tf(flop, t) if T > 32 else _gb(wbytes, t),
                                      ms=round(t * 1e3, 4))
        # the layer's steps one by one (each graph-replayed)
        off, gat, slot, rg = nv.moe_align(ids, E, gates)
        act = nv.grouped_gemm(x, gat, off, w1c, w1s, R, epilogue=nv.EPI_SWIGLU)
        y = nv.grouped_gemm(act, None, off, w2c, w2s, R, row_scale=rg)
        steps = {
            "align": (lambda: nv.moe_align(ids, E, gates), None),
            "gate_up": (lambda: nv.grouped_gemm(x, gat, off, w1c, w1s, R, epilogue=nv.EPI_SWIGLU,
                                                out=act), 2 * R * 1536 * 2048),
            "down": (lambda: nv.grouped_gemm(act, None, off, w2c, w2s, R, row_scale=rg, out=y),
                     2 * R * 2048 * 768),
            "combine": (lambda: nv.moe_combine(y, slot), None),
        }
        for name, (fn, fl) in steps.items():
            ts = timeit(fn)
            res[f"moe_T{T}_{name}_us"] = round(ts * 1e6, 2)
            if fl and T > 32:
                res[f"moe_T{T}_{name}"] = _tf(fl, ts)
        # the layer on expert weights tiled once (nvfp4_grouped_gemm_tiled)
        w1t, w2t = nv.tile_experts(w1c, w1s), nv.tile_experts(w2c, w2s)
        t = timeit(lambda: nv.moe_layer_tiled(x, ids, gates, w1t, w2t, E, 768))
        res[f"moe_tiled_T{T}_layer"] = dict(_tf(flop, t) if T > 32 else _gb(wbytes, t),
                                            ms=round(t * 1e3, 4))
        steps_t = {
            "gate_up": (lambda: nv.grouped_gemm_tiled(x, gat, off, w1t, E, 1536, R,
                                                      epilogue=nv.EPI_SWIGLU, out=act),
                        2 * R * 1536 * 2048),
            "down": (lambda: nv.grouped_gemm_tiled(act, None, off, w2t, E, 2048, R, row_scale=rg,
                                                   out=y), 2 * R * 2048 * 768),
        }
        for name, (fn, fl) in steps_t.items():
            ts = timeit(fn)
            res[f"moe_tiled_T{T}_{name}_us"] = round(ts * 1e6, 2)
            if T > 32:
                res[f"moe_tiled_T{T}_{name}"] = _tf(fl, ts)
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_configs(budget_s=4.0):
    """The oracle (as it stands) beside the GPU on the other configurations, each
    on a bounded, evenly spaced sample of its rows, scaled to the config's unit:
    prefill and W4A4 on 256 of 8192 / 512 activation rows (all weight rows),
    the quantizer on 512 rows, the MoE layer on 32 tokens (T = 32) and on 64 of
    4096 tokens (T = 4096)."""
    import oracle
    import workloads as wl
    res = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    for (K, N) in [(wl.HIDDEN, wl.MLP), (wl.MLP, wl.HIDDEN)]:
        x, w = wl.prefill(K, N)
        rows = np.linspace(0, 8191, 256).astype(np.int64)
        # calibrate on 8 rows, then as many rows as fit the budget (<= 256)
        t8 = timed(lambda: oracle.gemm_w4a16(np.ascontiguousarray(x[rows[:8]]), 8, K, w.codes,
                                             w.scales))
        n = int(min(256, max(8, 8 * budget_s / max(t8, 1e-3))))
        sel = np.ascontiguousarray(x[rows[:n]])
        t = timed(lambda: oracle.gemm_w4a16(sel, n, K, w.codes, w.scales))
        res[f"prefill_M8192_K{K}_N{N}"] = {
            "value": round(2 * n * N * K / t / 1e9, 3), "unit": "GFLOP/s",
            "sample": f"{n} of 8192 rows (evenly spaced), all {N} weight rows: {t:.2f} s"}
        del x, w
    x, w = wl.w4a4()
    t = timed(lambda: oracle.quantize(x, 512, wl.HIDDEN))
    res["quantize_M512_K5120"] = {"value": round(512 * wl.HIDDEN * (2 + 9 / 16) / t / 1e9, 4),
                                  "unit": "GB/s", "sample": f"all 512 rows: {t:.2f} s"}
    ac, as_ = oracle.quantize(x, 512, wl.HIDDEN)
    n = 32
    t = timed(lambda: oracle.gemm_w4a4(np.ascontiguousarray(ac[:n]), np.ascontiguousarray(as_[:n]),
                                       n, wl.HIDDEN, w.codes, w.scales))
    res["w4a4_M512_N17408_K5120"] = {"value": round(2 * n * wl.MLP * wl.HIDDEN / t / 1e9, 3),
                                     "unit": "GFLOP/s",
                                     "sample": f"{n} of 512 rows, all weight rows: {t:.2f} s"}
    for T, n_tok in ((32, 32), (4096, 64)):
        m = wl.moe(T)
        toks = np.linspace(0, T - 1, n_tok).astype(np.int64)
        t = timed(lambda: oracle.moe_layer(np.ascontiguousarray(m.x[toks]),
                                           np.ascontiguousarray(m.ids[toks]),
                                           np.ascontiguousarray(m.gates[toks]), 128, 768,
                                           m.w1.codes, m.w1.scales, m.w2.codes, m.w2.scales))
        res[f"moe_T{T}_layer"] = {
            "value": round(2 * n_tok * 8 * (1536 * 2048 + 2048 * 768) / t / 1e9, 3),
            "unit": "GFLOP/s", "sample": f"{n_tok} of {T} tokens: {t:.2f} s"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device-to-device copy 3 times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--case", action="append", choices=SECONDARY_CASES,
                    help="run only these secondary rows (no decode set); for profiling one "
                         "kernel at a time")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the NVFP4 layer is built for a single GPU "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_gemm_nvfp4_amd as nv
    nv.lib()  # raises if the HIP library is missing
    assert torch.cuda.is_available(), "no GPU visible"

    def dev_u8(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()

    def dev_bf16(b):
        return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).cuda().view(
            torch.bfloat16)

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    hd = (dev_u8, dev_bf16, dev_i32)
    if args.case:
        print(json.dumps({"cases": secondary(nv, torch, hd, cases=args.case)}), flush=True)
        return
    log("generating decode workload")
    dec = Decode(nv, torch, hd)
    # the clocks settle only after some sustained load: run the step for ~0.2 s
    # first (untimed), so the timed passes see the steady state
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for c in dec.calls:
            c[4]()
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps x {len(dec.calls)} calls (warmup {args.warmup}): "
        "eager with per-call events, then as a replayed graph")
    wall_eager, per_call = time_decode(dec, torch, args.steps, args.warmup)
    wall = time_decode_graph(dec, torch, args.steps, args.warmup)
    step_bytes = dec.step_bytes()
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes * args.steps / wall / 1e9
    eager_value = step_bytes * args.steps / wall_eager / 1e9

    # roofline of the decode GEMV kernel: algorithmic weight bytes per launch over
    # the mean launch time, from HIP events on the launch stream
    launch_bytes = np.array([weight_bytes(rows, K) for (_, _, K, rows, _) in dec.calls])
    mean_ms = per_call.mean(axis=0)
    achieved = float(launch_bytes.sum() / (mean_ms.sum() / 1e3) / 1e9)
    per_call_gbs = {c[0]: round(float(b / (t / 1e3) / 1e9), 1)
                    for c, b, t in zip(dec.calls, launch_bytes, mean_ms)}
    per_call_us = {c[0]: round(float(t * 1e3), 2) for c, t in zip(dec.calls, mean_ms)}
    draft = None
    if not args.no_secondary:
        log("secondary: masked head draft proposal (top-8)")
        draft = time_draft(dec, torch, nv)
    del dec
    torch.cuda.empty_cache()
    # the same step with every call on the row-major layout (nvfp4_gemm)
    log("the decode step on row-major weights (graph-replayed)")
    dec_r = Decode(nv, torch, hd, tiled=False)
    wall_r = time_decode_graph(dec_r, torch, args.steps, args.warmup)
    _, per_call_r = time_decode(dec_r, torch, args.steps, args.warmup)
    row_major = {
        "value_GBs": round(step_bytes * args.steps / wall_r / 1e9, 2),
        "ms_per_step": round(wall_r / args.steps * 1e3, 4),
        "per_call_us": {c[0]: round(float(t * 1e3), 2)
                        for c, t in zip(dec_r.calls, per_call_r.mean(axis=0))},
    }
    del dec_r
    torch.cuda.empty_cache()
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {COPY_PROBE_BYTES} bytes")
        del src, dst

    sec = None
    if not args.no_secondary:
        sec = secondary(nv, torch, hd)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline()
        cpu["cpu_model"] = cpu_model()
        if not args.no_secondary:
            log("oracle on the other configurations (bounded samples)")
            cpu["configs"] = cpu_configs()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; NVFP4 e2m1 codes + E4M3 scales, bf16 activations)",
        "config": {
            "workload": ("decode W4A16 GEMV set: M in {1,8,32} x (K,N) in {(5120,17408),"
                         "(17408,5120),(5120,248320)} + masked head 32768/248320 rows"),
            "step_weight_bytes": int(step_bytes),
            "calls_per_step": len(per_call_us),
            "step": ("12 nvfp4_gemm_tiled calls captured as one HIP graph, replayed, on "
                     "weights tiled once at load (nvfp4_tile_weight; the masked head's fixed "
                     "32,768-row id set tiled as its own matrix)"),
            "eager_GBs": round(eager_value, 2),
            "row_major": row_major,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes": int(step_bytes),
            "kernel": ("k_gemv4_tiled / k_gemv<TL> (decode GEMV on tiled weights, all 12 "
                       "launches of a step; bytes per step)"),
        },
        "per_call_GBs": per_call_gbs,
        "per_call_us": per_call_us,
    }
    if sec is not None:
        line["secondary"] = sec
    if draft is not None:
        line["draft_proposal"] = draft
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
