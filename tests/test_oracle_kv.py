"""Pins of the oracle's FP8 E4M3 KV-cache codec: the encoder against torch's
float8_e4m3fn cast (a library routine) on every bf16 value and on exact ties,
saturation and signed zero by definition, the decode round trip of every code;
the store path against numpy's binary32 division followed by that cast, and the
load path against numpy's binary32 product followed by torch's bf16 cast, with
the paging, padding and zero-fill rules on small cases worked by hand."""
import numpy as np
import torch

import helpers


def _torch_e4m3(q32):
    """float32 values with |q| <= 448 -> E4M3 codes by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(q32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _enc_all(orc, vals):
    return np.array([orc.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)


def test_encode_matches_torch_on_every_bf16_in_range(orc):
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    got = _enc_all(orc, f[keep].astype(np.float64))
    assert np.array_equal(got, _torch_e4m3(f[keep]))


def test_encode_ties_go_to_even_code(orc):
    t = helpers.e4m3_table_torch()
    codes = np.arange(0, 0x7E)
    mids = 0.5 * (t[codes] + t[codes + 1])          # exact midpoints
    got = _enc_all(orc, mids)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want)
    assert np.array_equal(_enc_all(orc, -mids), want | 0x80)
    assert np.array_equal(got, _torch_e4m3(mids.astype(np.float32)))


def test_encode_saturates_and_keeps_sign_of_zero(orc):
    for v in (448.0, 463.9, 464.0, 1e6, float(np.finfo(np.float32).max)):
        assert orc.e4m3_encode(v) == 0x7E and orc.e4m3_encode(-v) == 0xFE
    assert orc.e4m3_encode(0.0) == 0x00 and orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(2.0 ** -10) == 0x00          # tie between 0 and 2^-9
    assert orc.e4m3_encode(-(2.0 ** -11)) == 0x80


def test_decode_encode_round_trip_every_code(orc):
    t = helpers.e4m3_table_torch()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(_enc_all(orc, t[codes]), codes)


def _store_ref(x_bits, scale):
    """numpy binary32 division, then torch's cast (saturated by hand)."""
    x = helpers.bf16_bits_to_f64(x_bits).astype(np.float32)
    q = x / np.float32(scale)
    sat = np.abs(q) > 448.0
    codes = _torch_e4m3(np.where(sat, 0.0, q))
    codes[sat] = np.where(np.signbit(q[sat]), 0xFE, 0x7E)
    return codes


def test_store_matches_numpy_division_and_torch_cast(orc):
    rng = np.random.default_rng(31)
    T, W, slots = 37, 64, 80
    x = helpers.f64_to_bf16_bits_exact(
        torch.from_numpy(rng.standard_normal((T, W)) * 40).to(torch.bfloat16).double().numpy())
    x[0, :4] = [0x0000, 0x8000, 0x0001, 0x8001]          # signed zeros, bf16 subnormals
    slot = rng.permutation(slots)[:T].astype(np.int32)
    slot[3] = -1                                         # padding token
    for scale in (1.0, 0.0375, 3.3):
        cache = np.full((slots, W), 0xAA, dtype=np.uint8)
        orc.kv_store_e4m3(x, slot, scale, cache)
        ref = _store_ref(x, scale)
        for t in range(T):
            if slot[t] >= 0:
                assert np.array_equal(cache[slot[t]], ref[t]), (scale, t)
        untouched = np.setdiff1d(np.arange(slots), slot[slot >= 0])
        assert np.all(cache[untouched] == 0xAA)


def test_load_matches_numpy_product_and_torch_cast(orc):
    rng = np.random.default_rng(32)
    slots, W, page = 64, 32, 16
    cache = rng.integers(0, 256, size=(slots, W), dtype=np.uint8)
    cache[cache == 0x7F] = 0x7E
    cache[cache == 0xFF] = 0xFE
    bt = np.array([[3, 0, 2], [1, 3, 0]], dtype=np.int32)
    lens = np.array([40, 17], dtype=np.int32)
    scale = 0.0123
    out = orc.kv_load_e4m3(cache, bt, lens, page, 48, scale)
    t = helpers.e4m3_table_torch().astype(np.float32)
    for b in range(2):
        for i in range(48):
            if i >= lens[b]:
                assert np.all(out[b, i] == 0)
                continue
            s = bt[b, i // page] * page + i % page
            p = t[cache[s]] * np.float32(scale)
            want = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(out[b, i], want), (b, i)


def test_store_then_load_is_identity_on_e4m3_values(orc):
    """Inputs that are E4M3 values times a power-of-two scale come back exactly."""
    rng = np.random.default_rng(33)
    t = helpers.e4m3_table_torch()
    codes = rng.integers(0, 0x7E, size=(20, 16)) | (rng.integers(0, 2, size=(20, 16)) << 7)
    for scale in (1.0, 0.25, 8.0):
        x = helpers.f64_to_bf16_bits_exact(t[codes] * scale)
        cache = np.zeros((32, 16), dtype=np.uint8)
        orc.kv_store_e4m3(x, np.arange(20, dtype=np.int32) + 4, scale, cache)
        back = orc.kv_load_e4m3(cache, np.array([[0, 1]], np.int32), np.array([24], np.int32),
                                16, 24, scale)
        got = back[0, 4:24]
        assert np.array_equal(got & 0x7FFF, x & 0x7FFF)
        nz = (x & 0x7FFF) != 0
        assert np.array_equal(got[nz], x[nz])


def test_encode_nan_is_the_nan_code_of_its_sign(orc):
    """A NaN quotient becomes the format's NaN code with its sign (0x7F / 0xFF),
    as torch's float8_e4m3fn cast gives (a library routine); infinities keep the
    satfinite reading (448), where torch's cast would give NaN."""
    for bits in (0x7FC0, 0x7F81, 0xFFC0, 0xFFFF):
        v = float(helpers.bf16_bits_to_f64(np.array([bits], np.uint16))[0])
        want = int(_torch_e4m3(np.array([v], np.float32))[0])
        assert want == (0xFF if bits & 0x8000 else 0x7F)
        assert orc.e4m3_encode(v) == want
    assert orc.e4m3_encode(float("inf")) == 0x7E and orc.e4m3_encode(-float("inf")) == 0xFE


def test_store_nan_leaves_neighbours_exact(orc):
    """A NaN element of a token row gets its NaN code; every other element of the
    row and of the cache is what the store gives without it (nothing spills
    into the next code)."""
    rng = np.random.default_rng(12)
    T, W, slots = 4, 32, 8
    x = helpers.f64_to_bf16_bits_exact(
        helpers.bf16_bits_to_f64(((rng.standard_normal((T, W)).astype(np.float32).view(np.uint32)
                                   + 0x8000) >> 16).astype(np.uint16)))
    sm = np.array([5, 0, 7, 2], np.int32)
    base = orc.kv_store_e4m3(x, sm, 0.05, np.zeros((slots, W), np.uint8))
    xn = x.copy()
    xn[1, 9], xn[2, 0], xn[2, 31] = 0x7FC0, 0xFFC0, 0x7FC0
    got = orc.kv_store_e4m3(xn, sm, 0.05, np.zeros((slots, W), np.uint8))
    want = base.copy()
    want[0, 9], want[7, 0], want[7, 31] = 0x7F, 0xFF, 0x7F
    assert np.array_equal(got, want)
