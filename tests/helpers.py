"""Shared test helpers: golden-file parsers, an independent fp64 decoder built
from library routines (torch's float8_e4m3fn) and the golden e2m1 table, and
the GEMM tolerance check."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def e2m1_table():
    """16 e2m1 values from the golden file (float64, -0.0 kept)."""
    t = np.zeros(16)
    for line in golden_lines("e2m1_values.txt"):
        c, v = line.split()
        t[int(c)] = float(v)
    return t


def e4m3_table_torch():
    """All 256 E4M3 codes decoded by torch's float8_e4m3fn (a library routine)."""
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant_independent(codes, scales):
    """fp64 dequantization by table lookup (golden e2m1, torch E4M3)."""
    codes = np.asarray(codes)
    lo = codes & 15
    hi = codes >> 4
    el = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    vals = e2m1_table()[el]
    s = e4m3_table_torch()[np.asarray(scales)]
    s = np.repeat(s, 16, axis=-1)
    return vals * s


def bf16_bits_to_f64(b):
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_exact(v):
    """fp64 values that are exactly representable in bf16 -> bits."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64), equal_nan=True)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def all_bf16_nonneg_finite():
    """Every non-negative finite bf16 bit pattern (0x0000 .. 0x7F7F)."""
    return np.arange(0, 0x7F80, dtype=np.uint16)


def gemm_close(got, ref_f64, out_is_bf16=True, rel_frob=1e-3, elem=1e-2, abs_extra=None):
    """Tolerance of the GEMM outputs: relative Frobenius error <= 1e-3 and every
    element within 1e-2*(|ref|+1).  For a bf16 output the reference is the fp64
    sum rounded once to bf16 (the comparison an exact kernel would pass).
    abs_extra (same shape as ref, optional) widens each element's bound by that
    amount: the fp32 summation error bound K * 2^-24 * sum |terms| of sums whose
    terms cancel far below their magnitude (outside the stated workloads).
    Returns (ok, rel_frobenius, worst_element_ratio)."""
    import oracle
    ref = np.asarray(ref_f64, dtype=np.float64)
    if out_is_bf16:
        ref = bf16_bits_to_f64(oracle.bf16_round(ref))
        g = bf16_bits_to_f64(got)
    else:
        g = np.asarray(got, dtype=np.float64)
    if not np.all(np.isfinite(g)):
        return False, float("inf"), float("inf")
    diff = g - ref
    denom = np.linalg.norm(ref)
    rf = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    bound = elem * (np.abs(ref) + 1.0)
    if abs_extra is not None:
        bound = bound + np.asarray(abs_extra, dtype=np.float64)
    worst = float(np.max(np.abs(diff) / bound)) if diff.size else 0.0
    return (rf <= rel_frob and worst <= 1.0), rf, worst


# ---- GPU helpers (only used by tests marked gpu) ------------------------------------

def announce(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)


def dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits):
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t):
    """bf16 GPU tensor -> uint16 bit patterns (numpy)."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def topk_valid(vals, ids, logits_f64, row_idx, tol):
    """Whether (vals, ids) [M][k] is a valid draft proposal for exact logits
    logits_f64 [M][n] (columns are row_idx, or 0..n-1) when the proposer saw
    the logits with an error of at most tol: ids distinct and kept; each value
    within tol of its exact logit; values non-increasing; and no id's exact
    logit below the exact k-th best by more than 2*tol."""
    logits = np.asarray(logits_f64, dtype=np.float64)
    M, n = logits.shape
    cols_of = {int(r): c for c, r in enumerate(row_idx)} if row_idx is not None else None
    vals = np.asarray(vals, dtype=np.float64)
    for m in range(M):
        k = len(ids[m])
        if len(set(int(i) for i in ids[m])) != k:
            return False
        cols = []
        for i in ids[m]:
            c = cols_of.get(int(i)) if cols_of is not None else (int(i) if 0 <= int(i) < n else None)
            if c is None:
                return False
            cols.append(c)
        exact = logits[m, cols]
        if np.any(np.abs(vals[m] - exact) > tol):
            return False
        if np.any(np.diff(vals[m]) > 0):
            return False
        kth = np.sort(logits[m])[::-1][k - 1]
        if np.any(exact < kth - 2 * tol):
            return False
    return True


GUARD_BYTES = 4096


class Guarded:
    """A device output of `shape` and `dtype` with GUARD_BYTES of a fill
    pattern on each side.  `t` is the output tensor (contiguous, 16-byte
    aligned); check() asserts that no byte of either guard changed, i.e. the
    kernel wrote nothing past its output."""

    def __init__(self, shape, dtype):
        import torch
        n = 1
        for d in shape:
            n *= int(d)
        item = torch.empty((), dtype=dtype).element_size()
        self.nbytes = n * item
        pat = (np.arange(GUARD_BYTES) * 37 + 11) % 251
        self.pattern = torch.from_numpy(pat.astype(np.uint8))
        buf = torch.empty(2 * GUARD_BYTES + self.nbytes, dtype=torch.uint8, device="cuda")
        buf[:GUARD_BYTES] = self.pattern.cuda()
        buf[GUARD_BYTES + self.nbytes:] = self.pattern.cuda()
        self.buf = buf
        self.t = buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(*shape)

    def check(self):
        import torch
        torch.cuda.synchronize()
        lo = self.buf[:GUARD_BYTES].cpu()
        hi = self.buf[GUARD_BYTES + self.nbytes:].cpu()
        assert torch.equal(lo, self.pattern), "write before the start of the output"
        assert torch.equal(hi, self.pattern), "write past the end of the output"
