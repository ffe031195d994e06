"""GPU parity of the FP8 E4M3 KV-cache codec against the oracle: every result
is bit-exact (codes of the store, bf16 rows of the load)."""
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


def _store_gpu(nv, x, slot, scale, cache0):
    import torch
    cache = torch.from_numpy(cache0.copy()).cuda()
    nv.kv_store_e4m3(helpers.dev_bf16(x), helpers.dev_i32(slot), scale, cache)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0375, 3.3, 2.0 ** -20, 1.0e5])
def test_store_every_finite_bf16(nv, orc, scale):
    """All 65,280 finite bf16 values (both zeros, subnormals, the largest) under
    several scales, including ones that saturate or flush most of them."""
    helpers.announce(f"kv store every bf16 scale={scale}")
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = np.isfinite((bits << 16).view(np.float32))
    vals = bits[finite].astype(np.uint16)
    W = 1024
    T = (len(vals) + W - 1) // W
    x = np.zeros(T * W, dtype=np.uint16)
    x[:len(vals)] = vals
    x = x.reshape(T, W)
    slot = np.arange(T, dtype=np.int32)[::-1].copy()
    cache0 = np.full((T + 3, W), 0xAA, dtype=np.uint8)
    got = _store_gpu(nv, x, slot, scale, cache0)
    ref = orc.kv_store_e4m3(x, slot, scale, cache0.copy())
    assert np.array_equal(got, ref)


def test_store_padding_and_out_of_range_slots(nv, orc):
    helpers.announce("kv store padding slots")
    rng = np.random.default_rng(70)
    T, W, slots = 50, 48, 40
    x = workloads.normal_bf16(rng, T, W)
    slot = rng.permutation(64)[:T].astype(np.int32)   # some >= slots: skipped
    slot[::7] = -1
    cache0 = rng.integers(0, 256, size=(slots, W), dtype=np.uint8)
    got = _store_gpu(nv, x, slot, 0.02, cache0)
    ref = orc.kv_store_e4m3(x, slot, 0.02, cache0.copy())
    assert np.array_equal(got, ref)


def test_store_prefill_full_size_sampled(nv, orc):
    """8192 tokens x 1024 elements into 16-token pages, in the configuration the
    benchmark times; 256 stored rows recomputed by the oracle."""
    import torch
    helpers.announce("kv store T=8192 W=1024")
    w = workloads.kv_store(8192)
    cache = torch.zeros((w.num_slots, workloads.KV_W), dtype=torch.uint8, device="cuda")
    nv.kv_store_e4m3(helpers.dev_bf16(w.x), helpers.dev_i32(w.slot_mapping), w.scale, cache)
    got = cache.cpu().numpy()
    rows = np.sort(np.random.default_rng(71).choice(8192, 256, replace=False))
    sub = np.zeros((256, workloads.KV_W), dtype=np.uint8)
    orc.kv_store_e4m3(w.x[rows], np.arange(256, dtype=np.int32), w.scale, sub)
    assert np.array_equal(got[w.slot_mapping[rows]], sub)
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_mapping)
    assert np.all(got[untouched] == 0)


@pytest.mark.parametrize("B,max_len,W,page", [(1, 1, 16, 16), (3, 40, 64, 16), (5, 100, 128, 32),
                                              (2, 17, 32, 1)])
def test_load_matches_oracle(nv, orc, B, max_len, W, page):
    import torch
    helpers.announce(f"kv load B={B} max_len={max_len} W={W} page={page}")
    cache, bt, lens, scale = workloads.kv_load(B, max_len, W=W, page=page, seed=B + W)
    bt = bt.copy()
    if bt.size > 2:
        bt.flat[-1] = cache.shape[0] // page + 5          # a page outside the cache: zeros
    out = nv.kv_load_e4m3(helpers.dev_u8(cache), helpers.dev_i32(bt), helpers.dev_i32(lens),
                          page, max_len, scale)
    got = helpers.host_bits(out)
    ref = orc.kv_load_e4m3(cache, bt, lens, page, max_len, scale)
    assert np.array_equal(got, ref)
    torch.cuda.synchronize()


def test_load_decode_full_size_sampled(nv, orc):
    """32 sequences up to 4096 tokens x 1024 elements, 16-token pages: the
    benchmark's configuration; sampled sequences recomputed by the oracle."""
    helpers.announce("kv load B=32 max_len=4096 W=1024")
    B, L = 32, 4096
    cache, bt, lens, scale = workloads.kv_load(B, L)
    out = helpers.host_bits(nv.kv_load_e4m3(helpers.dev_u8(cache), helpers.dev_i32(bt),
                                            helpers.dev_i32(lens), workloads.KV_PAGE, L, scale))
    for b in (0, 7, 31):
        ref = orc.kv_load_e4m3(cache, bt[b:b + 1], lens[b:b + 1], workloads.KV_PAGE, L, scale)
        assert np.array_equal(out[b], ref[0]), b


def test_store_then_load_round_trip(nv, orc):
    """GPU store followed by GPU load equals the oracle's composition."""
    import torch
    helpers.announce("kv store+load round trip")
    w = workloads.kv_store(300, W=256, spare_pages=3, seed=5)
    cache = torch.zeros((w.num_slots, 256), dtype=torch.uint8, device="cuda")
    nv.kv_store_e4m3(helpers.dev_bf16(w.x), helpers.dev_i32(w.slot_mapping), w.scale, cache)
    pages = w.slot_mapping[::16] // 16
    bt = pages[None, :].astype(np.int32)
    lens = np.array([300], dtype=np.int32)
    out = helpers.host_bits(nv.kv_load_e4m3(cache, helpers.dev_i32(bt), helpers.dev_i32(lens), 16,
                                            304, w.scale))
    c_ref = orc.kv_store_e4m3(w.x, w.slot_mapping, w.scale,
                              np.zeros((w.num_slots, 256), dtype=np.uint8))
    ref = orc.kv_load_e4m3(c_ref, bt, lens, 16, 304, w.scale)
    assert np.array_equal(out, ref)


def test_store_nan_elements_confined(nv, orc):
    """NaN elements (both signs) become the NaN codes 0x7F / 0xFF; every other
    code of the cache is bit-exact against the oracle (no spill into the next
    code of the packed word)."""
    helpers.announce("kv store NaN elements")
    rng = np.random.default_rng(71)
    T, W, slots = 8, 64, 12
    x = workloads.normal_bf16(rng, T, W)
    x[0, 3], x[0, 4], x[5, 63], x[7, 0] = 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF
    slot = rng.permutation(slots)[:T].astype(np.int32)
    cache0 = rng.integers(0, 256, size=(slots, W), dtype=np.uint8)
    got = _store_gpu(nv, x, slot, 0.03, cache0)
    ref = orc.kv_store_e4m3(x, slot, 0.03, cache0.copy())
    assert ref[slot[0], 3] == 0x7F and ref[slot[0], 4] == 0xFF
    assert np.array_equal(got, ref)
