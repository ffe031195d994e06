"""Pins of the oracle's format decoders and rounding steps against things other
than itself: hand-derived golden values, torch's float8_e4m3fn / bfloat16 casts
(library routines), and exhaustive brute force with exact arithmetic."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import helpers


def test_e2m1_table_matches_golden(orc):
    """Oracle's bit-field e2m1 decode vs the 16 listed values (sign of zero too)."""
    for line in helpers.golden_lines("e2m1_values.txt"):
        c, v = line.split()
        got = orc.e2m1_value(int(c))
        want = float(v)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got, want)


def test_e4m3_golden_values(orc):
    for line in helpers.golden_lines("e4m3_values.txt"):
        c, v = line.split()
        got = orc.e4m3_value(int(c, 16))
        if v == "nan":
            assert math.isnan(got), c
        else:
            want = float(v)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got, want)


def test_e4m3_all_256_match_torch(orc):
    ref = helpers.e4m3_table_torch()
    for c in range(256):
        got = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c


def test_bf16_value_matches_torch(orc):
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_value(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_on_f32_inputs(orc):
    """For fp32-representable inputs torch's float->bfloat16 cast is a single
    nearest-even rounding, so it pins the oracle's rounding directly."""
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties: low half 0x8000 / 0x7FFF / 0x8001
    u[:3000] = (u[:3000] & 0xFFFF0000) | 0x8000
    u[3000:6000] = (u[3000:6000] & 0xFFFF0000) | 0x7FFF
    u[6000:9000] = (u[6000:9000] & 0xFFFF0000) | 0x8001
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_double_inputs_nearest_even(orc):
    """fp64 inputs that are not fp32 values: check nearest (exact Fractions) and
    the tie rule directly -- no library does one-step double->bf16."""
    rng = np.random.default_rng(12)
    vals = list(rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000)))
    # exact halfway points between adjacent bf16 values, plus a hair either side
    for b in rng.integers(1, 0x7F7F, 500):
        lo = helpers.bf16_bits_to_f64(np.uint16(b))
        hi = helpers.bf16_bits_to_f64(np.uint16(b + 1))
        mid = (lo + hi) / 2
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    vals = np.array(vals)
    got = orc.bf16_round(vals)
    for v, g in zip(vals, got):
        gv = Fraction(float(helpers.bf16_bits_to_f64(g)))
        fv = Fraction(float(v))
        s = 1 if v >= 0 else -1
        gb = int(g) & 0x7FFF
        nb_dn = helpers.bf16_bits_to_f64(np.uint16((gb - 1) | (int(g) & 0x8000))) if gb > 0 else None
        nb_up = helpers.bf16_bits_to_f64(np.uint16((gb + 1) | (int(g) & 0x8000)))
        d = abs(fv - gv)
        for nb in (nb_dn, nb_up):
            if nb is None or not math.isfinite(nb):
                continue
            dn = abs(fv - Fraction(float(nb)))
            assert d <= dn, (v, g)
            if d == dn:  # tie: the kept value has an even last bit
                assert gb % 2 == 0, (v, g)
        assert (g >> 15) == (1 if s < 0 else 0) or gv == 0


def _e4m3_finite_nonneg(orc):
    return np.array([orc.e4m3_value(c) for c in range(0x7F)])


def test_scale_rounding_exhaustive_brute_force(orc):
    """Every non-negative finite bf16 block maximum a: the scale code equals the
    candidate (of the 127 finite non-negative E4M3 values) nearest to a/6, ties to
    the even code -- found by brute force over all candidates.  Distances are
    compared as |a - 6v|, exact in fp64 for a in [2^-10, 2^13]; below that a/6 is
    under half the smallest subnormal (code 0), above it a/6 > 1365 (code 0x7E)."""
    a = helpers.bf16_bits_to_f64(helpers.all_bf16_nonneg_finite())
    got = orc.scale_codes(a)
    v = _e4m3_finite_nonneg(orc)
    want = np.empty_like(got)
    lo = a < 2.0**-10
    hi = a > 2.0**13
    mid = ~(lo | hi)
    want[lo] = 0
    want[hi] = 0x7E
    am = a[mid]
    d = np.abs(am[:, None] - 6.0 * v[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    codes = np.arange(0x7F)
    # among tied candidates keep the even code
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10**6).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 10**6).min(axis=1)
    ntie = cand.sum(axis=1)
    want[mid] = np.where(ntie > 1, even_pick, any_pick)
    assert np.array_equal(got, want)
    assert (ntie > 1).sum() > 0  # the sweep does contain exact ties


def test_scale_rounding_matches_torch_cast_in_range(orc):
    """In range (a/6 <= 448), torch's fp32 -> float8_e4m3fn cast (nearest even) of
    fp32(a/6) must give the same code."""
    a = helpers.bf16_bits_to_f64(helpers.all_bf16_nonneg_finite())
    t = (a.astype(np.float32) / np.float32(6.0))
    keep = t <= 448.0
    ref = torch.from_numpy(t[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.scale_codes(a[keep])
    assert np.array_equal(got, ref)


def test_code_rounding_exhaustive_brute_force(orc):
    """Every finite bf16 x against every finite non-negative scale code: the code is
    sign(x) | index of the e2m1 magnitude nearest to |x|/s (ties to the even
    index), found by brute force over the 8 magnitudes with exact fp64 distances
    |x| - s*v (exact for s/64 <= |x| <= 2^20; below s/64 the nearest is 0, above
    2^20 > 6*448 it is 6).  Scale 0 gives magnitude 0."""
    pos = helpers.all_bf16_nonneg_finite()
    bits = np.concatenate([pos, pos | np.uint16(0x8000)])
    ax = helpers.bf16_bits_to_f64(pos)
    ax = np.concatenate([ax, ax])
    sign = np.concatenate([np.zeros(len(pos), np.uint8), np.full(len(pos), 8, np.uint8)])
    mags = np.abs(helpers.e2m1_table()[:8])
    idx = np.arange(8)
    n_ties = 0
    for sc in range(0x7F):
        s = orc.e4m3_value(sc)
        got = orc.e2m1_encodes(bits, sc)
        if s == 0.0:
            want = sign.copy()
        else:
            m = np.empty(len(ax), dtype=np.uint8)
            small = ax < s / 64
            big = ax > 2.0**20
            mid = ~(small | big)
            m[small] = 0
            m[big] = 7
            d = np.abs(ax[mid][:, None] - s * mags[None, :])
            cand = d == d.min(axis=1, keepdims=True)
            nt = cand.sum(axis=1)
            n_ties += int((nt > 1).sum())
            even_pick = np.where(cand & (idx[None, :] % 2 == 0), idx[None, :], 99).min(axis=1)
            any_pick = np.where(cand, idx[None, :], 99).min(axis=1)
            m[mid] = np.where(nt > 1, even_pick, any_pick)
            want = sign | m
        assert np.array_equal(got, want), hex(sc)
    assert n_ties > 0


def test_quantize_golden_blocks(orc):
    for line in helpers.golden_lines("quantize_blocks.txt"):
        name, vals, sc, codes = [p.strip() for p in line.split("|")]
        x = helpers.f64_to_bf16_bits_exact([float(v) for v in vals.split()])
        want_codes = [int(c, 16) for c in codes.split()]
        # K must be a multiple of 32 in the library; the oracle accepts 16.  Pad with a
        # second all-zero block so the row is 32 wide.
        xx = np.concatenate([x, np.zeros(16, np.uint16)]).reshape(1, 32)
        qc, qs = orc.quantize(xx, 1, 32)
        assert qs[0, 0] == int(sc, 16), (name, hex(qs[0, 0]))
        got = []
        for j in range(8):
            got += [int(qc[0, j]) & 15, int(qc[0, j]) >> 4]
        assert got == want_codes, (name, got)
        assert qs[0, 1] == 0 and np.all(qc[0, 8:] == 0)


def test_quantize_roundtrip(orc):
    """Blocks whose codes include a +-6 and any non-zero finite scale code:
    dequantize, then quantize again -> identical codes and scale (amax = 6s gives
    a/6 = s exactly and every element sits exactly on the grid)."""
    rng = np.random.default_rng(3)
    nb = 4000
    codes16 = rng.integers(0, 16, size=(nb, 16))
    pos = rng.integers(0, 16, size=nb)
    codes16[np.arange(nb), pos] = rng.choice([7, 15], size=nb)
    sc = rng.integers(1, 0x7F, size=nb).astype(np.uint8)
    packed = (codes16[:, 0::2] | (codes16[:, 1::2] << 4)).astype(np.uint8)
    # one block per row, padded to K = 32 with a second block of zeros
    codes = np.concatenate([packed, np.zeros((nb, 8), np.uint8)], axis=1)
    scales = np.stack([sc, np.zeros(nb, np.uint8)], axis=1)
    deq = orc.dequantize(codes, scales, nb, 32)
    qc, qs = orc.quantize(deq, nb, 32)
    assert np.array_equal(qs[:, 0], sc)
    assert np.array_equal(qc[:, :8], packed)


def test_amax_maps_to_six_for_normal_scales(orc):
    """If a block's scale is an E4M3 normal (code >= 0x08), the element holding the
    block maximum gets magnitude 6 (index 7): a/s lies within (5.6, 6.4) or
    saturates.  Checked for every bf16 block maximum."""
    a_bits = helpers.all_bf16_nonneg_finite()
    a = helpers.bf16_bits_to_f64(a_bits)
    sc = orc.scale_codes(a)
    normal = sc >= 0x08
    assert normal.sum() > 10000
    for c in np.unique(sc[normal]):
        sel = a_bits[normal & (sc == c)]
        got = orc.e2m1_encodes(sel, int(c))
        assert np.all(got == 7), hex(c)


def test_quantize_error_bound(orc):
    """|x - deq(q(x))| <= half the local grid gap times s for |x| <= 6s, and the
    error of saturated elements is |x| - 6s."""
    rng = np.random.default_rng(4)
    M, K = 64, 256
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-12, 10, (M, 1)))).astype(np.float32)
    xb = helpers.f64_to_bf16_bits_exact(
        helpers.bf16_bits_to_f64(((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)))
    xb = xb.reshape(M, K)
    qc, qs = orc.quantize(xb, M, K)
    deq = helpers.bf16_bits_to_f64(orc.dequantize(qc, qs, M, K))
    xv = helpers.bf16_bits_to_f64(xb)
    s = np.repeat(helpers.e4m3_table_torch()[qs], 16, axis=1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    gaps = np.diff(grid)
    ax = np.abs(xv)
    r = np.where(s > 0, ax / np.where(s > 0, s, 1), 0)
    seg = np.clip(np.searchsorted(grid, r, side="right") - 1, 0, 6)
    bound = np.where(r <= 6, 0.5 * gaps[seg] * s, ax - 6 * s)
    err = np.abs(xv - deq)
    ok = (err <= bound + 0.0) | (s == 0)
    assert ok.all()
    # with a zero scale every element is below 6 * 2^-10 and is stored as zero
    assert np.all(ax[s == 0] <= 6 * 2.0**-10)


def test_nan_block_is_confined(orc):
    """Non-finite inputs are outside the quantizer's contract, but a block that
    holds a NaN stays confined to itself: its scale is the E4M3 NaN code 0x7F
    and its codes keep only their sign bits; every other block of the row is
    exactly what it is without the NaN block.  An infinite element saturates
    (scale 0x7E, magnitude index 7)."""
    assert orc.scale_code(float("nan")) == 0x7F
    assert orc.scale_code(float("inf")) == 0x7E
    rng = np.random.default_rng(5)
    x = helpers.f64_to_bf16_bits_exact(
        helpers.bf16_bits_to_f64(((rng.standard_normal((2, 64)).astype(np.float32).view(np.uint32)
                                   + 0x8000) >> 16).astype(np.uint16)))
    qc0, qs0 = orc.quantize(x, 2, 64)
    xn = x.copy()
    xn[0, 20] = 0x7FC0      # NaN in block 1 of row 0
    xn[1, 63] = 0xFFC0      # -NaN in block 3 of row 1
    qc, qs = orc.quantize(xn, 2, 64)
    assert qs[0, 1] == 0x7F and qs[1, 3] == 0x7F
    keep = np.ones((2, 4), bool)
    keep[0, 1] = keep[1, 3] = False
    assert np.array_equal(qs[keep], qs0[keep])
    nib = np.stack([qc & 15, qc >> 4], axis=-1).reshape(2, 64)
    nib0 = np.stack([qc0 & 15, qc0 >> 4], axis=-1).reshape(2, 64)
    sign = ((xn >> 15) & 1).astype(np.uint8) << 3
    for r, b in ((0, 1), (1, 3)):
        assert np.array_equal(nib[r, 16 * b:16 * b + 16], sign[r, 16 * b:16 * b + 16])
    other = np.repeat(keep, 16, axis=1)
    assert np.array_equal(nib[other], nib0[other])
    xi = x.copy()
    xi[0, 0] = 0x7F80       # +inf
    qc, qs = orc.quantize(xi, 2, 64)
    assert qs[0, 0] == 0x7E and (qc[0, 0] & 15) == 7
