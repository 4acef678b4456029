"""Pins for the oracle's align/permute: invariants, closed forms, brute force."""
import numpy as np
import pytest

import oracle


def brute_force_layout(ids: np.ndarray, E: int, B: int, cap: int):
    flat = ids.reshape(-1)
    R = flat.size
    rows, experts = [], []
    for e in range(E):
        items = [r for r in range(R) if flat[r] == e]
        padded = items + [R] * ((-len(items)) % B)
        rows += padded
        experts += [e] * (len(padded) // B)
    npp = len(rows)
    sorted_ids = np.array(rows + [R] * (cap - npp), np.int32)
    expert_ids = np.array(experts + [-1] * (cap // B - len(experts)), np.int32)
    return sorted_ids, expert_ids, npp


def check_invariants(ids, E, B, sorted_ids, expert_ids, npp, inv):
    flat = ids.reshape(-1)
    R = flat.size
    counts = np.bincount(flat, minlength=E)
    assert npp == int(sum((c + B - 1) // B * B for c in counts))      # closed form
    assert npp % B == 0
    real = sorted_ids[:npp][sorted_ids[:npp] < R]
    assert np.array_equal(np.sort(real), np.arange(R))                  # a permutation
    assert np.all(sorted_ids[npp:] == R) and np.all(expert_ids[npp // B:] == -1)
    assert np.all(np.diff(expert_ids[:npp // B]) >= 0)                  # experts ascend
    for b in range(npp // B):
        blk = sorted_ids[b * B:(b + 1) * B]
        items = blk[blk < R]
        assert np.all(flat[items] == expert_ids[b])                     # one expert per block
    for e in range(E):                                                   # ascending r, then pads
        seg = sorted_ids[:npp][np.repeat(expert_ids[:npp // B], B) == e]
        n = counts[e]
        assert np.all(np.diff(seg[:n]) > 0) and np.all(seg[n:] == R)
    assert np.array_equal(sorted_ids[inv.reshape(-1)], np.arange(R))    # inverse permutation


@pytest.mark.parametrize("M,k,E,B", [(64, 2, 8, 16), (32, 8, 128, 16), (100, 4, 16, 32),
                                     (7, 3, 5, 64), (300, 8, 256, 128), (500, 2, 6, 256)])
def test_align_random(M, k, E, B):
    g = np.random.default_rng(M + k + E + B)
    ids = np.stack([g.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
    cap = oracle.align_capacity(M, k, E, B)
    s, x, npp, inv = oracle.align(ids, E, B)
    check_invariants(ids, E, B, s, x, npp, inv)
    bs, bx, bnpp = brute_force_layout(ids, E, B, cap)
    assert npp == bnpp and np.array_equal(s, bs) and np.array_equal(x, bx)
    assert npp <= cap


def test_align_skewed_and_empty_experts():
    g = np.random.default_rng(11)
    M, k, E, B = 200, 4, 64, 16
    # only 5 experts ever chosen, one of them by every token
    ids = np.stack([np.r_[0, g.choice(np.arange(1, 5), k - 1, replace=False)] for _ in range(M)])
    ids = ids.astype(np.int32)
    s, x, npp, inv = oracle.align(ids, E, B)
    check_invariants(ids, E, B, s, x, npp, inv)
    assert set(x[:npp // B]) <= {0, 1, 2, 3, 4}


def test_align_capacity_bound_is_tight_for_worst_case():
    # every expert receives one item: R + E*(B-1) rows, the bound exactly
    M, k, E, B = 16, 4, 64, 16
    ids = np.arange(M * k, dtype=np.int32).reshape(M, k) % E
    cap = oracle.align_capacity(M, k, E, B)
    s, x, npp, inv = oracle.align(ids, E, B)
    assert npp == cap == E * B


def test_align_empty():
    ids = np.zeros((0, 2), np.int32)
    assert oracle.align_capacity(0, 2, 8, 16) == 0
    s, x, npp, inv = oracle.align(ids, 8, 16)
    assert npp == 0 and s.size == 0 and x.size == 0
