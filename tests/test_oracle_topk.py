"""Pins of the oracle's draft proposal (top-k over the masked head's logits):
hand-worked orders, numpy's sorting routines on random and tie-heavy rows,
argmax for k = 1, the row-index map, and the head composed with an independent
decoder on one-hot activations (whose logits are the weights themselves)."""
import numpy as np
import pytest

import helpers
import workloads


def _golden():
    for line in helpers.golden_lines("topk_order.txt"):
        vals, k, cols = [p.strip() for p in line.split("|")]
        yield (np.array([float(t) for t in vals.split()]), int(k),
               np.array([int(t) for t in cols.split()]))


def test_topk_hand_worked_orders(orc):
    for v, k, cols in _golden():
        got_v, got_i = orc.topk(v[None, :], k)
        assert got_i[0].tolist() == cols.tolist(), (v, k)
        assert np.array_equal(np.signbit(got_v[0]), np.signbit(v[cols]))
        assert np.array_equal(got_v[0], v[cols])


def test_topk_random_rows_match_stable_argsort(orc):
    rng = np.random.default_rng(21)
    v = rng.standard_normal((5, 3000)).astype(np.float32)
    for k in (1, 7, 64, 3000):
        got_v, got_i = orc.topk(v, k)
        ref = np.argsort(-v.astype(np.float64), axis=1, kind="stable")[:, :k]
        assert np.array_equal(got_i, ref)
        assert np.array_equal(got_v, np.take_along_axis(v, ref, 1))


def test_topk_tie_heavy_rows_match_lexsort(orc):
    """Values from a small set with +-0 and +-inf: numpy's lexsort with keys
    (value descending, +0 before -0, column ascending)."""
    rng = np.random.default_rng(22)
    pool = np.array([-np.inf, -2.0, -0.5, -0.0, 0.0, 0.5, 1.0, 1.0, 3.0, np.inf])
    v = pool[rng.integers(0, len(pool), size=(6, 777))]
    k = 100
    got_v, got_i = orc.topk(v, k)
    cols = np.arange(v.shape[1])
    for m in range(v.shape[0]):
        order = np.lexsort((cols, np.signbit(v[m]), -v[m]))[:k]
        assert np.array_equal(got_i[m], order)
        assert np.array_equal(np.signbit(got_v[m]), np.signbit(v[m][order]))


def test_topk_one_is_first_argmax(orc):
    rng = np.random.default_rng(23)
    v = rng.integers(-4, 5, size=(9, 500)).astype(np.float64)  # many ties, no -0
    _, got_i = orc.topk(v, 1)
    assert np.array_equal(got_i[:, 0], np.argmax(v, axis=1))


def test_topk_ids_map_and_bounds(orc):
    rng = np.random.default_rng(24)
    v = rng.standard_normal((3, 50))
    idx = np.sort(rng.choice(1000, 50, replace=False)).astype(np.int32)
    _, cols = orc.topk(v, 10)
    _, ids = orc.topk(v, 10, ids_map=idx)
    assert np.array_equal(ids, idx[cols])
    with pytest.raises(ValueError):
        orc.topk(v, 51)
    with pytest.raises(ValueError):
        orc.topk(v, 0)


def test_head_topk_one_hot_rows_select_weight_column(orc):
    """With x = e_j the logit of kept row r is w[r][j] exactly, so the proposal is
    the top-k of one weight column (decoded independently) over the mask."""
    rng = np.random.default_rng(25)
    N, K, n_keep, k = 700, 64, 300, 16
    w = workloads.nvfp4_weight(rng, N, K)
    idx = np.sort(rng.choice(N, n_keep, replace=False)).astype(np.int32)
    js = [0, 5, 33, 63]
    x = np.zeros((len(js), K), dtype=np.float64)
    x[np.arange(len(js)), js] = 1.0
    xb = helpers.f64_to_bf16_bits_exact(x)
    vals, ids, logits = orc.head_topk(xb, len(js), K, w.codes, w.scales, k, row_idx=idx)
    W = helpers.dequant_independent(w.codes, w.scales)
    for m, j in enumerate(js):
        col = W[idx, j]
        order = np.lexsort((np.arange(n_keep), np.signbit(col), -col))[:k]
        assert np.array_equal(ids[m], idx[order])
        assert np.array_equal(vals[m], col[order])


def test_topk_validity_check_detects_errors(orc):
    """The check applied to GPU proposals from rounded logits accepts the exact
    answer and rejects a duplicated id, an id outside the mask, an id whose
    logit is far below the k-th best, a wrong value and a wrong order."""
    rng = np.random.default_rng(26)
    logits = rng.standard_normal((2, 400))
    idx = np.sort(rng.choice(5000, 400, replace=False)).astype(np.int32)
    k, tol = 8, 1e-6
    v, ids = orc.topk(logits, k, ids_map=idx)
    assert helpers.topk_valid(v, ids, logits, idx, tol)
    bad = ids.copy(); bad[0, 1] = bad[0, 0]
    assert not helpers.topk_valid(v, bad, logits, idx, tol)
    bad = ids.copy(); bad[1, 3] = 4999 if 4999 not in idx else 4998
    assert not helpers.topk_valid(v, bad, logits, idx, tol)
    worst = idx[np.argmin(logits[0])]
    bad = ids.copy(); bad[0, k - 1] = worst
    assert not helpers.topk_valid(v, bad, logits, idx, tol)
    badv = v.copy(); badv[1, 2] += 1e-3
    assert not helpers.topk_valid(badv, ids, logits, idx, tol)
    assert not helpers.topk_valid(v[:, ::-1], ids[:, ::-1], logits, idx, tol)
