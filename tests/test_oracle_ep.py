"""Pins for the oracle's expert-parallel shard (an expert map from global ids
to this rank's experts, -1 for experts held elsewhere).

* Align with a map equals a brute-force layout of the items whose expert is
  local, renumbered through the map; remote items get no row.
* The identity map reduces to the unsharded oracle bit for bit.
* Sharding invariance: splitting the experts over G ranks, each holding only
  its experts' weights, the ranks' unrounded fp64 accumulators sum to the
  unsharded accumulator (the same terms, regrouped).
* A rank that holds none of the chosen experts outputs exactly zero.
"""
import numpy as np
import pytest

import oracle
import synth
from hostutil import bits16, bits8
from test_oracle_align import check_invariants


def brute_force_ep(ids, emap, E_local, B, cap):
    flat = ids.reshape(-1)
    R = flat.size
    rows, experts = [], []
    inv = np.full(R, -1, np.int64)
    for e in range(E_local):
        items = [r for r in range(R) if emap[flat[r]] == e]
        for i, r in enumerate(items):
            inv[r] = len(rows) + i
        padded = items + [R] * ((-len(items)) % B)
        rows += padded
        experts += [e] * (len(padded) // B)
    npp = len(rows)
    s = np.array(rows + [R] * (cap - npp), np.int32)
    x = np.array(experts + [-1] * (cap // B - len(experts)), np.int32)
    return s, x, npp, inv.reshape(ids.shape)


def random_map(g, E_global, E_local):
    """E_local experts, chosen at random among E_global, with shuffled local ids."""
    emap = np.full(E_global, -1, np.int32)
    held = g.choice(E_global, E_local, replace=False)
    emap[held] = g.permutation(E_local)
    return emap


@pytest.mark.parametrize("M,k,Eg,El,B", [(64, 2, 8, 3, 16), (40, 8, 128, 16, 16), (300, 8, 256, 32, 128),
                                         (7, 3, 5, 5, 64), (200, 4, 16, 1, 32)])
def test_align_with_map_brute_force(M, k, Eg, El, B):
    g = np.random.default_rng(M + k + Eg + El)
    ids = np.stack([g.choice(Eg, k, replace=False) for _ in range(M)]).astype(np.int32)
    emap = random_map(g, Eg, El)
    cap = oracle.align_capacity(M, k, El, B)
    s, x, npp, inv = oracle.align(ids, El, B, expert_map=emap)
    bs, bx, bnpp, binv = brute_force_ep(ids, emap, El, B, cap)
    assert npp == bnpp <= cap
    assert np.array_equal(s, bs) and np.array_equal(x, bx) and np.array_equal(inv, binv)


def test_align_identity_map_is_the_plain_layout():
    g = np.random.default_rng(3)
    ids = np.stack([g.choice(16, 4, replace=False) for _ in range(100)]).astype(np.int32)
    plain = oracle.align(ids, 16, 32)
    mapped = oracle.align(ids, 16, 32, expert_map=np.arange(16, dtype=np.int32))
    for a, b in zip(plain, mapped):
        assert np.array_equal(a, b)
    check_invariants(ids, 16, 32, *plain)


def test_align_nothing_local():
    ids = np.array([[0, 1], [2, 3]], np.int32)
    for emap in (np.full(4, -1, np.int32), np.array([5, 7, -3, 9], np.int32)):  # out of range: remote
        s, x, npp, inv = oracle.align(ids, 4, 16, expert_map=emap)
        assert npp == 0 and np.all(inv == -1) and np.all(x == -1) and np.all(s == 4)


def test_align_global_id_out_of_range_raises():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 8]], np.int32), 2, 16, expert_map=np.zeros(8, np.int32))


def layer(fp8, p, inp, ids, w, sel=None, emap=None, on_input=False):
    sel = slice(None) if sel is None else sel
    if fp8:
        return oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q)[sel], inp.w13s.numpy()[sel],
                                        bits8(inp.w2q)[sel], inp.w2s.numpy()[sel], ids, w,
                                        on_input=on_input, return_acc=True, expert_map=emap)
    return oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13)[sel], bits16(inp.w2)[sel], ids, w,
                                     on_input=on_input, return_acc=True, expert_map=emap)


@pytest.mark.parametrize("fp8", [False, True])
def test_identity_map_layer_is_the_plain_layer(fp8):
    p = synth.Problem(M=9, H=256, I=256, E=6, topk=2, wdtype="fp8" if fp8 else "bf16")
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), p.topk)
    y0, a0 = layer(fp8, p, inp, ids, w)
    y1, a1 = layer(fp8, p, inp, ids, w, emap=np.arange(p.E, dtype=np.int32))
    assert np.array_equal(y0, y1) and np.array_equal(a0, a1)


@pytest.mark.parametrize("fp8,on_input,strided", [(False, False, False), (False, True, True),
                                                  (True, False, True)])
def test_sharded_accumulators_sum_to_the_full_layer(fp8, on_input, strided):
    p = synth.Problem(M=12, H=256, I=256, E=8, topk=3, wdtype="fp8" if fp8 else "bf16")
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), p.topk)
    _, full = layer(fp8, p, inp, ids, w, on_input=on_input)
    G = 4
    total = np.zeros_like(full)
    for rank in range(G):
        held = np.arange(rank, p.E, G) if strided else np.arange(rank * p.E // G, (rank + 1) * p.E // G)
        emap = np.full(p.E, -1, np.int32)
        emap[held] = np.arange(held.size)
        y, acc = layer(fp8, p, inp, ids, w, sel=held, emap=emap, on_input=on_input)
        total += acc
    assert np.allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())
    assert np.abs(full).max() > 0


def test_rank_holding_no_chosen_expert_outputs_zero():
    p = synth.Problem(M=5, H=256, I=128, E=4, topk=2)
    inp = synth.make_inputs(p, "cpu")
    ids = np.array([[0, 1]] * p.M, np.int32)
    w = np.full((p.M, 2), 0.5, np.float32)
    emap = np.array([-1, -1, 0, 1], np.int32)   # this rank holds experts 2 and 3
    y, acc = layer(False, p, inp, ids, w, sel=np.array([2, 3]), emap=emap)
    assert np.all(y == 0) and np.all(acc == 0)
