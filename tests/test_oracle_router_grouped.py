"""Pins for the oracle's grouped / sigmoid router.

* Reductions: one group (or keeping every group) with softmax scoring, no bias
  and scale 1 is the plain router, bit for bit.
* Sigmoid scoring: the ids are the plain top-k (sigmoid increases with the
  logit); the weights agree with scipy's expit in float64.
* Worked examples by hand (below), where a wrong group score (the largest key
  instead of the two largest with a bias, or the biased score as the weight)
  gives different ids or weights.
* A large bias forces an expert in and its weight stays its unbiased score; a
  strongly negative group is never kept; a power-of-two scale multiplies the
  weights exactly; renormalised weights sum to the scale.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def logits(M, E, seed):
    return np.random.default_rng(seed).standard_normal((M, E)).astype(np.float32)


@pytest.mark.parametrize("G,TG", [(1, 1), (8, 8), (4, 4)])
def test_reduces_to_the_plain_router(G, TG):
    s = logits(50, 64, 1)
    for renorm in (True, False):
        ids, w = oracle.topk(s, 6, renormalize=renorm)
        gi, gw = oracle.topk_grouped(s, 6, "softmax", renorm, G, TG)
        assert np.array_equal(ids, gi) and np.array_equal(w, gw)


def test_sigmoid_scores():
    s = logits(40, 32, 2)
    ids, _ = oracle.topk(s, 4)
    gi, gw = oracle.topk_grouped(s, 4, "sigmoid", renormalize=False)
    assert np.array_equal(ids, gi)
    sig = expit(np.take_along_axis(s.astype(np.float64), gi, 1))
    assert np.abs(gw - sig).max() < 1e-7
    _, rw = oracle.topk_grouped(s, 4, "sigmoid", renormalize=True)
    assert np.abs(rw - sig / sig.sum(1, keepdims=True)).max() < 1e-6


def test_worked_example_with_bias():
    # all logits 0: every sigmoid score is exactly 0.5. Keys 0.5 + bias:
    #   experts  0    1    2    3    4    5     6     7
    #   key     0.6  0.7  0.5  0.5  0.8  0.0  0.55  0.55
    # groups of 2: sums of the two best keys 1.3, 1.0, 0.8, 1.1 -> keep groups 0 and 3
    # (by the single best key it would be groups 2 and 0); the best two keys there
    # are experts 1 and 0; weights 0.5 and 0.5, renormalised 0.5 each, times 2.5.
    b = np.array([0.1, 0.2, 0.0, 0.0, 0.3, -0.5, 0.05, 0.05], np.float32)
    ids, w = oracle.topk_grouped(np.zeros((1, 8), np.float32), 2, "sigmoid", True, 4, 2, b, 2.5)
    assert ids.tolist() == [[1, 0]]
    assert w.tolist() == [[1.25, 1.25]]
    ids, w = oracle.topk_grouped(np.zeros((1, 8), np.float32), 3, "sigmoid", False, 4, 2, b, 1.0)
    assert ids.tolist() == [[1, 0, 6]] and w.tolist() == [[0.5, 0.5, 0.5]]  # 6 before 7: tie, lower index


def test_worked_example_without_bias():
    # no bias: a group's score is its largest logit. Groups of 4:
    #   group 0: 3.0, -5, -5, -5   (best 3.0)   group 1: 2.0, 1.9, 1.8, 1.7 (best 2.0)
    #   group 2: 2.5, 0, 0, 0      (best 2.5)   group 3: 0 ...
    # keep 2 groups: 0 and 2; top-3 among them: 3.0 (e0), 2.5 (e8), 0.0 (e9, lowest
    # index among the zeros), although group 1 holds four larger logits
    s = np.array([[3, -5, -5, -5, 2.0, 1.9, 1.8, 1.7, 2.5, 0, 0, 0, 0, 0, 0, 0]], np.float32)
    ids, _ = oracle.topk_grouped(s, 3, "softmax", True, 4, 2)
    assert ids.tolist() == [[0, 8, 9]]
    plain, _ = oracle.topk(s, 3)
    assert plain.tolist() == [[0, 8, 4]]


def test_bias_selects_but_does_not_weight():
    s = logits(30, 32, 3)
    b = np.zeros(32, np.float32)
    b[13] = 100.0
    ids, w = oracle.topk_grouped(s, 4, "sigmoid", False, 8, 2, b)
    assert np.all(ids[:, 0] == 13)
    assert np.abs(w[:, 0] - expit(s[:, 13].astype(np.float64))).max() < 1e-7
    b = np.zeros(32, np.float32)
    b[8:12] = -100.0                       # group 2 can never win
    ids, _ = oracle.topk_grouped(s, 4, "sigmoid", True, 8, 3, b)
    assert not np.any((ids >= 8) & (ids < 12))
    assert np.all(np.array([len(set(r // 4)) for r in ids]) <= 3)


def test_scale_and_sum():
    s = logits(20, 64, 4)
    b = np.random.default_rng(5).normal(0, 0.1, 64).astype(np.float32)
    _, w1 = oracle.topk_grouped(s, 8, "sigmoid", True, 8, 4, b, 1.0)
    _, w4 = oracle.topk_grouped(s, 8, "sigmoid", True, 8, 4, b, 4.0)
    assert np.array_equal(w4, w1 * 4)
    assert np.abs(w1.sum(1) - 1).max() < 1e-6


def test_invalid_arguments():
    s = logits(2, 16, 6)
    for kw in (dict(num_expert_group=3), dict(num_expert_group=4, topk_group=5),
               dict(num_expert_group=4, topk_group=1, k=5), dict(bias=np.zeros(16, np.float32)),
               dict(scoring="sigmoid", num_expert_group=16, bias=np.zeros(16, np.float32))):
        k = kw.pop("k", 2)
        with pytest.raises(ValueError):
            oracle.topk_grouped(s, k, **kw)
