"""Exact pins of the 8-bit layers' scale wiring in the oracle.

The step GEMMs are pinned on their own (test_oracle_ffn.py, test_oracle_mx.py);
these tests pin how the layers pick each expert's and each block's scales
("fused_moe.py analysis", "FP8 W8A8": one scale per 128x128 weight block and per
token per 128 activation columns; "DeepGEMM FusedMoE on Blackwell", TL;DR and
2.6.2: MXFP8 and W4A8 with one E8M0 scale per 32 values). The inputs spread
the scales over many powers of two (synth's scale_spread), so a scale taken
from the wrong expert, block or group moves results by large factors:

* every output is within a derived bound of the float64 layer on the
  dequantised weights (quant_bound.py), and the bound is not vacuous. These
  checks clear the sign bits of x and of the weight codes: with no cancellation
  in the sums the worst-case bound is a few percent of each value, where a
  scale that is off by a power of two moves it by tens of percent;
* the same check fails for the oracle run on planted mistakes: two experts'
  scale tensors swapped, each expert given its neighbour's scales, a transposed
  block grid, and the K blocks of the scales rotated by one;
* exact: doubling w2's scales of one expert and one 128-row block changes the
  fp64 accumulator only in that block's columns, only for tokens routed to that
  expert, and there by exactly alpha times that expert's output (taken from a
  top-1 call with weight 1).
"""
import numpy as np
import pytest

import oracle
import synth
from hostutil import bf16_f64, bits16, bits8
import quant_bound as qb


def routed(p):
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), p.topk)
    return inp, ids, w


def nonneg_bf16(x):
    return x & np.uint16(0x7FFF)


def nonneg_codes(q, fp4=False):
    """e4m3 codes: bit 7 is the sign; packed E2M1: bit 3 of each nibble."""
    return q & np.uint8(0x77 if fp4 else 0x7F)


def fp8_args(inp, positive=True):
    f = nonneg_codes if positive else (lambda q: q)
    return f(bits8(inp.w13q)), inp.w13s.numpy(), f(bits8(inp.w2q)), inp.w2s.numpy()


def mx_args(inp, fp4, positive=True):
    f = (lambda q: nonneg_codes(q, fp4)) if positive else (lambda q: q)
    return f(bits8(inp.w13q)), inp.w13s.numpy(), f(bits8(inp.w2q)), inp.w2s.numpy()


def run_fp8(x, w13q, w13s, w2q, w2s, ids, w, on_input=False, **kw):
    return oracle.fused_experts_fp8(x, w13q, w13s, w2q, w2s, ids, w, on_input=on_input, **kw)


FP8_CASES = [
    dict(M=12, H=256, I=256, E=4, topk=2),
    dict(M=9, H=384, I=256, E=3, topk=3, apply_router_weight_on_input=True),
    dict(M=10, H=256, I=384, E=5, topk=2),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_fp8_layer_within_derived_bound(cfg):
    p = synth.Problem(**cfg, wdtype="fp8", scale_spread=4, seed=21)
    inp, ids, w = routed(p)
    x = nonneg_bf16(bits16(inp.x))
    w13q, w13s, w2q, w2s = fp8_args(inp)
    on = p.apply_router_weight_on_input
    y = run_fp8(x, w13q, w13s, w2q, w2s, ids, w, on)
    W13, W2 = qb.deq_fp8_block(w13q, w13s), qb.deq_fp8_block(w2q, w2s)
    ref, bound = qb.layer_reference(bf16_f64(x), ids, w, W13, W2, qb.FP8_128, on)
    worst = qb.check(bf16_f64(y), ref, bound, str(cfg))
    assert worst > 0.02, worst            # the bound is not vacuous

    # planted mistakes in the scale wiring all leave the bound
    E = p.E
    swap = np.arange(E)
    swap[[0, 1]] = swap[[1, 0]]
    nb = np.roll(np.arange(E), 1)         # every expert reads its neighbour's scales
    plants = {
        "w13 scales of experts 0, 1 swapped": (w13s[swap], w2s),
        "w2 scales of experts 0, 1 swapped": (w13s, w2s[swap]),
        "each expert reads its neighbour's w13 scales": (w13s[nb], w2s),
        "each expert reads its neighbour's w2 scales": (w13s, w2s[nb]),
        "w13 scale K blocks rotated": (np.roll(w13s, 1, 2), w2s),
        "w2 scale row blocks rotated": (w13s, np.roll(w2s, 1, 1)),
    }
    if w2s.shape[1] == w2s.shape[2]:
        plants["w2 scale grid transposed"] = (w13s, np.ascontiguousarray(w2s.transpose(0, 2, 1)))
    for what, (s13, s2) in plants.items():
        bad = run_fp8(x, w13q, np.ascontiguousarray(s13), w2q, np.ascontiguousarray(s2), ids, w, on)
        assert qb.violates(bf16_f64(bad), ref, bound), f"planted mistake passed: {what}"


def test_fp8_doubling_one_w2_block_is_exact():
    p = synth.Problem(M=16, H=384, I=256, E=4, topk=2, wdtype="fp8", scale_spread=4, seed=22)
    inp, ids, w = routed(p)
    x = bits16(inp.x)
    w13q, w13s, w2q, w2s = fp8_args(inp, positive=False)
    _, acc = run_fp8(x, w13q, w13s, w2q, w2s, ids, w, return_acc=True)
    e, nb = 2, 1
    s2 = w2s.copy()
    s2[e, nb, :] *= 2.0
    _, acc2 = run_fp8(x, w13q, w13s, w2q, s2, ids, w, return_acc=True)
    d = acc2 - acc
    cols = np.zeros(p.H, bool)
    cols[nb * 128:(nb + 1) * 128] = True
    routed_to_e = (ids == e).any(1)
    assert routed_to_e.any() and (~routed_to_e).any()
    assert np.all(d[~routed_to_e] == 0.0)
    assert np.all(d[:, ~cols] == 0.0)
    for t in np.nonzero(routed_to_e)[0]:
        j = int(np.nonzero(ids[t] == e)[0][0])
        # expert e's output for token t alone: a top-1 call with weight 1 returns it as acc
        _, o = run_fp8(x[t:t + 1], w13q, w13s, w2q, w2s, np.array([[e]], np.int32),
                       np.ones((1, 1), np.float32), return_acc=True)
        want = float(w[t, j]) * o[0, cols]
        np.testing.assert_allclose(d[t, cols], want, rtol=1e-12, atol=0)
        assert np.abs(want).max() > 0


MX_CASES = [
    dict(M=10, H=256, I=256, E=4, topk=2, wdtype="mxfp8"),
    dict(M=8, H=384, I=256, E=3, topk=2, wdtype="mxfp8", apply_router_weight_on_input=True),
    dict(M=10, H=256, I=256, E=4, topk=2, wdtype="w4a8"),
    dict(M=8, H=256, I=384, E=3, topk=3, wdtype="w4a8", apply_router_weight_on_input=True),
]


@pytest.mark.parametrize("cfg", MX_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_mx_layer_within_derived_bound(cfg):
    p = synth.Problem(**cfg, scale_spread=4, seed=23)
    w4 = p.wdtype == "w4a8"
    inp, ids, w = routed(p)
    x = nonneg_bf16(bits16(inp.x))
    w13q, w13e, w2q, w2e = mx_args(inp, w4)
    on = p.apply_router_weight_on_input
    run = lambda a, b: oracle.fused_experts_mx(x, w13q, np.ascontiguousarray(a), w2q,
                                               np.ascontiguousarray(b), ids, w, w4=w4, on_input=on)
    y = run(w13e, w2e)
    W13, W2 = qb.deq_mx(w13q, w13e, w4), qb.deq_mx(w2q, w2e, w4)
    act = qb.FP8_128 if w4 else qb.MX_32
    ref, bound = qb.layer_reference(bf16_f64(x), ids, w, W13, W2, act, on)
    worst = qb.check(bf16_f64(y), ref, bound, str(cfg))
    assert worst > 0.02, worst
    E = p.E
    swap = np.arange(E)
    swap[[0, 1]] = swap[[1, 0]]
    nb = np.roll(np.arange(E), 1)
    plants = {
        "w13 codes of experts 0, 1 swapped": (w13e[swap], w2e),
        "w2 codes of experts 0, 1 swapped": (w13e, w2e[swap]),
        "each expert reads its neighbour's w13 codes": (w13e[nb], w2e),
        "each expert reads its neighbour's w2 codes": (w13e, w2e[nb]),
        "w13 codes' K blocks rotated": (np.roll(w13e, 1, 2), w2e),
        "w2 codes' K blocks rotated": (w13e, np.roll(w2e, 1, 2)),
        "w2 codes' rows rotated by 128": (w13e, np.roll(w2e, 128, 1)),
    }
    for what, (a, b) in plants.items():
        assert qb.violates(bf16_f64(run(a, b)), ref, bound), f"planted mistake passed: {what}"


@pytest.mark.parametrize("wdtype", ["mxfp8", "w4a8"])
def test_mx_doubling_one_w2_row_is_exact(wdtype):
    p = synth.Problem(M=12, H=256, I=256, E=3, topk=2, wdtype=wdtype, scale_spread=4, seed=24)
    w4 = wdtype == "w4a8"
    inp, ids, w = routed(p)
    x = bits16(inp.x)
    w13q, w13e, w2q, w2e = mx_args(inp, w4, positive=False)
    run = lambda b, ii=ids, ww=w, xx=x: oracle.fused_experts_mx(xx, w13q, w13e, w2q, b, ii, ww, w4=w4,
                                                                return_acc=True)[1]
    acc = run(w2e)
    e, rows = 1, [5, 130, 255]
    b = w2e.copy()
    b[e, rows, :] += 1                    # E8M0 code + 1: the row's scales double
    d = run(b) - acc
    routed_to_e = (ids == e).any(1)
    assert routed_to_e.any() and (~routed_to_e).any()
    assert np.all(d[~routed_to_e] == 0.0)
    other = np.ones(p.H, bool)
    other[rows] = False
    assert np.all(d[:, other] == 0.0)
    for t in np.nonzero(routed_to_e)[0]:
        j = int(np.nonzero(ids[t] == e)[0][0])
        o = run(w2e, np.array([[e]], np.int32), np.ones((1, 1), np.float32), x[t:t + 1])
        np.testing.assert_allclose(d[t, rows], float(w[t, j]) * o[0, rows], rtol=1e-12, atol=0)


def test_batched_fp8_within_derived_bound():
    rng = np.random.default_rng(25)
    p = synth.Problem(M=24, H=256, I=256, E=4, topk=1, wdtype="fp8", scale_spread=4, seed=25)
    inp = synth.make_inputs(p, "cpu")
    max_M = 6
    a = nonneg_bf16(bits16(inp.x)).reshape(p.E, max_M, p.H)
    counts = np.array([6, 0, 3, 8], np.int32)     # full, empty, partial, over-full
    w13q, w13s, w2q, w2s = fp8_args(inp)
    out = oracle.batched_experts_fp8(a, counts, w13q, w13s, w2q, w2s)
    W13, W2 = qb.deq_fp8_block(w13q, w13s), qb.deq_fp8_block(w2q, w2s)
    ref, bound = qb.batched_reference(bf16_f64(a), counts, W13, W2, qb.FP8_128)
    worst = qb.check(bf16_f64(out), ref, bound, "batched fp8")
    assert worst > 0.02, worst
    swap = np.array([2, 1, 0, 3])
    for what, (s13, s2) in {"w13 scales of experts 0, 2 swapped": (w13s[swap], w2s),
                            "w2 scales of experts 0, 2 swapped": (w13s, w2s[swap]),
                            "w2 scale row blocks rotated": (w13s, np.roll(w2s, 1, 1))}.items():
        bad = oracle.batched_experts_fp8(a, counts, w13q, np.ascontiguousarray(s13), w2q,
                                         np.ascontiguousarray(s2))
        assert qb.violates(bf16_f64(bad), ref, bound), f"planted mistake passed: {what}"
    del rng


def test_ep_fp8_layer_within_derived_bound():
    # an expert-parallel rank: local weights, global ids through the map
    p = synth.Problem(M=14, H=256, I=256, E=8, topk=2, wdtype="fp8", scale_spread=4, seed=26,
                      ep_size=2, ep_rank=1)
    inp, ids, w = routed(p)
    emap = inp.expert_map.numpy()
    x = nonneg_bf16(bits16(inp.x))
    w13q, w13s, w2q, w2s = fp8_args(inp)
    y = oracle.fused_experts_fp8(x, w13q, w13s, w2q, w2s, ids, w, expert_map=emap)
    W13, W2 = qb.deq_fp8_block(w13q, w13s), qb.deq_fp8_block(w2q, w2s)
    ref, bound = qb.layer_reference(bf16_f64(x), ids, w, W13, W2, qb.FP8_128, expert_map=emap)
    qb.check(bf16_f64(y), ref, bound, "EP rank fp8")
    swap = np.array([1, 0, 2, 3])
    bad = oracle.fused_experts_fp8(x, w13q, np.ascontiguousarray(w13s[swap]), w2q, w2s, ids, w, expert_map=emap)
    assert qb.violates(bf16_f64(bad), ref, bound)
