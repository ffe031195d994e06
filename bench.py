#!/usr/bin/env python3
"""Benchmark of the NVFP4 linear layer on one MI355X.

Workload of the headline metric (weight-stream GB/s at M = 1..32): the
decode-shaped W4A16 set -- M in {1, 8, 32} x (K, N) in {(5120, 17408),
(17408, 5120), (5120, 248320)} plus the masked head (32,768 of the 248,320
rows) -- 12 nvfp4_gemm calls.  One step runs all 12 calls once; `value` is the
weight bytes the step streams (rows * K * 9/16 per call) divided by the step
time, with every input resident in HBM before the timed region starts.  The
step is captured once as a HIP graph and replayed (as a serving engine replays
its decode step); the same calls launched one by one give config.eager_GBs and
the per-call event times of the roofline.

Infinity-cache (MALL, 256 MB) hygiene: dense weights exist in two copies and
the head in two copies; calls alternate copies and the masked head always
reads the copy the full head did not just read, so no call re-reads weights
that are still cached.

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
                   GB/s, MoE layer T=32 / T=4096);
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
    """The 12-call decode set with its weight copies, all resident on the GPU."""

    def __init__(self, nv, torch, helpers_dev):
        import workloads as wl
        self.nv, self.torch = nv, torch
        dev_u8, dev_bf16, dev_i32 = helpers_dev
        self.calls = []  # (name, M, K, rows, fn)
        shapes = wl.DECODE_SHAPES
        self.weights = {}
        for (K, N) in shapes:
            w = wl.decode_weights(K, N)
            copies = [(dev_u8(w.codes), dev_u8(w.scales))]
            copies.append((copies[0][0].clone(), copies[0][1].clone()))
            self.weights[(K, N)] = copies
            del w
        self.idx = dev_i32(wl.decode_masked_rows())
        self.x = {(M, K): dev_bf16(wl.decode_activations(M, K))
                  for M in wl.DECODE_M for K in {s[0] for s in shapes}}
        self.keep = []
        head = (wl.HIDDEN, wl.VOCAB)
        call_no = 0
        for M in wl.DECODE_M:
            for (K, N) in shapes:
                c = call_no % 2
                self._add(f"M{M}_K{K}_N{N}", M, K, N, self.weights[(K, N)][c], None, N)
                call_no += 1
            # masked head: the copy the full head call of this M did not read
            K, N = head
            c_full = (call_no - 1) % 2
            self._add(f"M{M}_masked_head", M, K, N, self.weights[head][1 - c_full], self.idx,
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


def secondary(nv, torch, helpers_dev, reps=3):
    """Single-GPU timings of the other rows of the layer (GPU events)."""
    import workloads as wl
    dev_u8, dev_bf16, dev_i32 = helpers_dev
    res = {}

    def timeit(fn, n=reps, warm_s=0.03, timed_s=0.03):
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

    # prefill GEMM, M = 8192
    for (K, N) in [(wl.HIDDEN, wl.MLP), (wl.MLP, wl.HIDDEN)]:
        log(f"secondary: prefill K={K} N={N}")
        x, w = wl.prefill(K, N)
        xd, wc, ws = dev_bf16(x), dev_u8(w.codes), dev_u8(w.scales)
        del x, w
        out = torch.empty((8192, N), dtype=torch.bfloat16, device="cuda")
        wsz = nv.gemm_workspace_size(8192, N, K, N)
        wsb = torch.empty(max(wsz, 1), dtype=torch.uint8, device="cuda")
        t = timeit(lambda: nv.gemm(xd, wc, ws, out=out, workspace=wsb), n=1)
        res[f"prefill_M8192_K{K}_N{N}_tflops"] = round(2 * 8192 * N * K / t / 1e12, 2)
        del xd, wc, ws, out, wsb
    # quantizer and W4A4 GEMM
    log("secondary: quantize + W4A4")
    x, w = wl.w4a4()
    xd = dev_bf16(x)
    t = timeit(lambda: nv.quantize(xd), n=20)
    res["quantize_M512_K5120_GBs"] = round(512 * 5120 * (2 + 9 / 16) / t / 1e9, 2)
    xq = dev_bf16(wl.normal_bf16(np.random.default_rng(0), 8192, 5120, 0.001))
    t = timeit(lambda: nv.quantize(xq), n=20)
    res["quantize_M8192_K5120_GBs"] = round(8192 * 5120 * (2 + 9 / 16) / t / 1e9, 2)
    codes, scales = nv.quantize(xd)
    wc, ws = dev_u8(w.codes), dev_u8(w.scales)
    t = timeit(lambda: nv.gemm(codes, wc, ws, a_scales=scales))
    res["w4a4_M512_N17408_K5120_tflops"] = round(2 * 512 * 17408 * 5120 / t / 1e12, 2)
    # W4A4 from bf16 activations with the quantizer fused in (decode shape)
    for M in (1, 8, 32):
        xm = dev_bf16(wl.normal_bf16(np.random.default_rng(M), M, wl.HIDDEN, 0.001))
        om = torch.empty((M, wl.MLP), dtype=torch.bfloat16, device="cuda")
        t_f = timeit(lambda: nv.gemm_w4a4(xm, wc, ws, out=om), n=20)

        def unfused():
            ac, as_ = nv.quantize(xm)
            nv.gemm(ac, wc, ws, a_scales=as_, out=om)
        t_u = timeit(unfused, n=20)
        res[f"w4a4_fused_M{M}_K5120_N17408_us"] = round(t_f * 1e6, 2)
        res[f"w4a4_quantize_then_gemm_M{M}_K5120_N17408_us"] = round(t_u * 1e6, 2)
    del xd, xq, wc, ws
    # two-level NVFP4: offline weight quantizer (amax pass + quantize pass)
    log("secondary: offline weight quantizer")
    wq = dev_bf16(wl.normal_bf16(np.random.default_rng(1), wl.MLP, wl.HIDDEN))
    wqs = torch.empty(nv.lib().nvfp4_quantize_weight_workspace_size(wl.MLP, wl.HIDDEN),
                      dtype=torch.uint8, device="cuda")
    t = timeit(lambda: nv.quantize_weight(wq, workspace=wqs), n=10)
    res["quantize_weight_N17408_K5120_GBs"] = round(
        wl.MLP * wl.HIDDEN * (2 + 2 + 9 / 16) / t / 1e9, 1)   # two reads of bf16, codes + scales out
    del wq, wqs
    # FP8 E4M3 KV-cache codec: bytes moved (bf16 in + codes out; codes in + bf16 out)
    log("secondary: KV cache store / load")
    kw = wl.kv_store(8192)
    kx, ksm = dev_bf16(kw.x), dev_i32(kw.slot_mapping)
    kc = torch.zeros((kw.num_slots, wl.KV_W), dtype=torch.uint8, device="cuda")
    t = timeit(lambda: nv.kv_store_e4m3(kx, ksm, kw.scale, kc), n=20)
    res["kv_store_T8192_W1024_GBs"] = round(8192 * wl.KV_W * 3 / t / 1e9, 1)
    cache, bt, lens, kscale = wl.kv_load(32, 4096)
    kc2, kbt, kl = dev_u8(cache), dev_i32(bt), dev_i32(lens)
    kout = torch.empty((32, 4096, wl.KV_W), dtype=torch.bfloat16, device="cuda")
    t = timeit(lambda: nv.kv_load_e4m3(kc2, kbt, kl, wl.KV_PAGE, 4096, kscale, out=kout), n=10)
    used = int(lens.sum()) * wl.KV_W
    res["kv_load_B32_L4096_W1024_GBs"] = round((used * 3 + (32 * 4096 * wl.KV_W - used) * 2)
                                               / t / 1e9, 1)
    del kx, ksm, kc, kc2, kbt, kl, kout, cache
    # MoE layer
    for T in (32, 4096):
        log(f"secondary: MoE T={T}")
        m = wl.moe(T)
        args = (dev_bf16(m.x), dev_i32(m.ids), torch.from_numpy(m.gates).cuda(),
                dev_u8(m.w1.codes), dev_u8(m.w1.scales), dev_u8(m.w2.codes), dev_u8(m.w2.scales))
        t = timeit(lambda: nv.moe_layer(*args))
        touched = len(np.unique(m.ids))
        if T == 32:
            b = touched * (1536 * 2048 + 2048 * 768) * 9 // 16
            res["moe_T32_weight_GBs"] = round(b / t / 1e9, 2)
        res[f"moe_T{T}_tflops"] = round(2 * T * 8 * (1536 * 2048 + 2048 * 768) / t / 1e12, 3)
        res[f"moe_T{T}_ms"] = round(t * 1e3, 3)
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
    cpu = None if args.no_cpu else cpu_baseline()

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
            "step": "12 nvfp4_gemm calls captured as one HIP graph, replayed",
            "eager_GBs": round(eager_value, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes": int(step_bytes),
            "kernel": "k_gemv / k_gemv4 (decode GEMV, all 12 launches of a step; bytes per step)",
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
