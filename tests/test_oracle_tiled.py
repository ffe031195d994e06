"""Pins of the oracle's tiled weight layout (oracle.tile_weight): offsets worked
by hand from the layout's definition (tests/golden/tiled_layout.txt), the zero
padding of rows past N and elements past K, the size, and that a whole-tile
matrix is a byte permutation of its codes and scales."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiled_layout.txt")


def _marked(N, K):
    """Codes and scales whose bytes are non-zero and differ between neighbours."""
    r = np.arange(N)[:, None]
    codes = ((7 * r + 3 * np.arange(K // 2)[None, :] + 1) % 255 + 1).astype(np.uint8)
    scales = ((5 * r + 11 * np.arange(K // 16)[None, :] + 2) % 254 + 1).astype(np.uint8)
    return codes, scales


def _golden():
    shape, entries, zeros = None, [], []
    for line in open(GOLDEN):
        f = line.split("#")[0].split()
        if not f:
            continue
        if f[0] == "shape":
            shape = (int(f[1]), int(f[2]))
        elif f[0] in ("code", "scale"):
            entries.append((f[0], int(f[1]), int(f[2]), int(f[3])))
        elif f[0] == "zero":
            zeros.append((int(f[1]), int(f[2])))
    return shape, entries, zeros


def test_hand_worked_offsets():
    (N, K), entries, zeros = _golden()
    codes, scales = _marked(N, K)
    t = oracle.tile_weight(codes, scales, N, K)
    assert t.size == 4 * 2304
    for kind, r, j, off in entries:
        src = codes[r, j] if kind == "code" else scales[r, j]
        assert t[off] == src, f"{kind}[{r}][{j}] expected at {off}"
    for lo, hi in zeros:
        assert not t[lo:hi].any(), f"bytes [{lo}, {hi}) must be zero"


@pytest.mark.parametrize("N,K", [(1, 32), (17, 288), (16, 256), (40, 544), (3, 5120)])
def test_size_and_padding(N, K):
    codes, scales = _marked(N, K)
    t = oracle.tile_weight(codes, scales, N, K)
    T, S = -(-N // 16), -(-K // 256)
    assert t.size == T * S * 2304
    # the non-zero bytes are exactly the (non-zero) input bytes
    assert np.count_nonzero(t) == codes.size + scales.size


@pytest.mark.parametrize("N,K", [(16, 256), (32, 512), (48, 1024)])
def test_whole_tiles_are_a_permutation(N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
    t = oracle.tile_weight(codes, scales, N, K)
    assert t.size == N * K * 9 // 16
    assert np.array_equal(np.sort(t), np.sort(np.concatenate([codes.ravel(), scales.ravel()])))


def test_row_and_step_blocks_are_contiguous():
    """One tile's K range is contiguous: changing row 5 only changes bytes of
    tile 0; changing element 300 of row 20 only changes block (1, 1)."""
    N, K = 40, 544
    codes, scales = _marked(N, K)
    base = oracle.tile_weight(codes, scales, N, K)
    S = 3
    c2 = codes.copy()
    c2[5, :] ^= 0xFF
    d = np.nonzero(oracle.tile_weight(c2, scales, N, K) != base)[0]
    assert d.size == K // 2 and d.min() >= 0 and d.max() < S * 2304
    c3 = codes.copy()
    c3[20, 150] ^= 0x0F  # elements 300, 301
    d = np.nonzero(oracle.tile_weight(c3, scales, N, K) != base)[0]
    assert d.size == 1 and (1 * S + 1) * 2304 <= d[0] < (1 * S + 2) * 2304
