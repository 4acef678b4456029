"""Pins for the oracle's router: softmax over all experts, top-k, renormalise.

Checked against brute-force sorting, closed forms and scipy's softmax.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


@pytest.mark.parametrize("M,E,k", [(50, 8, 2), (40, 256, 8), (30, 128, 8), (20, 16, 16), (10, 5, 1)])
def test_topk_brute_force(M, E, k):
    g = np.random.default_rng(M * 1000 + E)
    logits = g.standard_normal((M, E)).astype(np.float32)
    ids, w = oracle.topk(logits, k)
    for t in range(M):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert list(ids[t]) == order
        p = softmax(logits[t].astype(np.float64))
        sel = p[order] / p[order].sum()
        np.testing.assert_allclose(w[t], sel, rtol=3e-7, atol=0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 4 * 2.0 ** -24 * k


def test_topk_without_renormalisation_is_softmax():
    g = np.random.default_rng(5)
    logits = g.standard_normal((16, 32)).astype(np.float32)
    ids, w = oracle.topk(logits, 4, renormalize=False)
    for t in range(16):
        p = softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=3e-7)


def test_topk_two_closed_form():
    g = np.random.default_rng(6)
    logits = (g.standard_normal((64, 8)) * 3).astype(np.float32)
    ids, w = oracle.topk(logits, 2)
    for t in range(64):
        s0, s1 = float(logits[t, ids[t, 0]]), float(logits[t, ids[t, 1]])
        assert s0 >= s1
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(s1 - s0))) <= 1e-7
        assert abs(w[t, 1] - 1.0 / (1.0 + math.exp(s0 - s1))) <= 1e-7


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_topk_all_equal_logits(k):
    logits = np.full((3, 16), 0.75, np.float32)
    ids, w = oracle.topk(logits, k)
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (3, 1)))
    assert np.all(w == np.float32(1.0 / k))


def test_topk_ties_go_to_lower_index():
    logits = np.array([[0.0, 2.0, 1.0, 2.0, 1.0, 2.0]], np.float32)
    ids, _ = oracle.topk(logits, 4)
    assert list(ids[0]) == [1, 3, 5, 2]


def test_topk_k_equals_e_is_sorted_softmax():
    g = np.random.default_rng(7)
    logits = g.standard_normal((8, 12)).astype(np.float32)
    ids, w = oracle.topk(logits, 12)
    for t in range(8):
        p = softmax(logits[t].astype(np.float64))
        assert sorted(ids[t]) == list(range(12))
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=3e-7)
        assert np.all(np.diff(w[t]) <= 0)


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros((2, 4), np.float32), 5)


def test_topk_nan_logits_rank_below_every_number():
    # reading: a NaN logit counts as -inf (never chosen over a number, lower index
    # first among such, softmax term 0); a row with no number has NaN weights
    g = np.random.default_rng(8)
    logits = g.standard_normal((6, 16)).astype(np.float32)
    logits[0, [0, 3, 9]] = np.nan                 # a few NaNs: never chosen with k = 4
    logits[1, :14] = np.nan                       # two numbers left, k = 4: NaN ids 0, 1 follow
    logits[2, :] = np.nan                         # no number: ids 0..3, weights NaN
    logits[3, 5] = -np.inf
    logits[3, 6] = np.nan                         # -inf (5) before NaN (6) only by index
    for renorm in (True, False):
        ids, w = oracle.topk(logits, 4, renormalize=renorm)
        mapped = np.where(np.isnan(logits), -np.inf, logits).astype(np.float64)
        for t in range(6):
            order = sorted(range(16), key=lambda e: (-mapped[t, e], e))[:4]
            assert list(ids[t]) == order
        assert not np.isin(ids[0], [0, 3, 9]).any()
        assert list(ids[1]) == ([14, 15, 0, 1] if logits[1, 14] >= logits[1, 15] else [15, 14, 0, 1])
        assert list(ids[2]) == [0, 1, 2, 3] and np.isnan(w[2]).all()
        for t in (0, 1, 3, 4, 5):
            assert np.isfinite(w[t]).all()
            p = softmax(mapped[t])
            ref = p[ids[t]] / p[ids[t]].sum() if renorm else p[ids[t]]
            np.testing.assert_allclose(w[t], ref, rtol=3e-7, atol=0)
        assert w[1, 2] == 0.0 and w[1, 3] == 0.0   # the NaN experts' weights


def test_topk_grouped_nan_logits_rank_below_every_number():
    g = np.random.default_rng(9)
    logits = g.standard_normal((4, 32)).astype(np.float32)
    logits[0, [1, 2, 17]] = np.nan
    logits[1, 8:] = np.nan
    bias = (g.standard_normal(32) * 0.05).astype(np.float32)
    ids, w = oracle.topk_grouped(logits, 4, "sigmoid", True, 4, 2, bias, 2.5)
    ids0, w0 = oracle.topk_grouped(np.where(np.isnan(logits), -np.inf, logits).astype(np.float32),
                                   4, "sigmoid", True, 4, 2, bias, 2.5)
    assert np.array_equal(ids, ids0) and np.array_equal(w, w0)
    assert np.all((ids >= 0) & (ids < 32))
    assert not np.isin(ids[0], [1, 2, 17]).any()
