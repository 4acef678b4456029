"""Pins for the oracle's batched-experts form ([E, max_M, H] batches, one per
expert, with per-expert counts; unweighted outputs).

* A batch row holds one routed item's token; with top-1 routing and weight 1
  the routed layer's output row is that item's expert output exactly (the
  weighted fp64 sum of one bf16 value times 1 rounds back to it), so the
  batched oracle on rows gathered per expert must equal the routed oracle
  bit for bit, for bf16 and fp8 weights.
* Rows at or past an expert's count are 0; an expert with count 0 outputs 0.
"""
import numpy as np
import pytest

import oracle
import synth
from hostutil import bits16, bits8


def batched_from_routing(x_bits, ids, E, max_M):
    """Gather each expert's tokens (ascending) into its batch."""
    a = np.zeros((E, max_M, x_bits.shape[1]), np.uint16)
    counts = np.zeros(E, np.int32)
    where = []
    for t, e in enumerate(ids[:, 0]):
        a[e, counts[e]] = x_bits[t]
        where.append((e, counts[e]))
        counts[e] += 1
    return a, counts, where


@pytest.mark.parametrize("fp8", [False, True])
def test_batched_equals_routed_top1(fp8):
    p = synth.Problem(M=24, H=256, I=256, E=5, topk=1, wdtype="fp8" if fp8 else "bf16")
    inp = synth.make_inputs(p, "cpu")
    ids, _ = oracle.topk(inp.logits.numpy(), 1)
    ones = np.ones((p.M, 1), np.float32)
    x = bits16(inp.x)
    max_M = int(np.bincount(ids[:, 0], minlength=p.E).max()) + 3   # spare rows stay 0
    a, counts, where = batched_from_routing(x, ids, p.E, max_M)
    if fp8:
        args = (bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q), inp.w2s.numpy())
        y = oracle.fused_experts_fp8(x, *args, ids, ones)
        out = oracle.batched_experts_fp8(a, counts, *args)
    else:
        y = oracle.fused_experts_bf16(x, bits16(inp.w13), bits16(inp.w2), ids, ones)
        out = oracle.batched_experts_bf16(a, counts, bits16(inp.w13), bits16(inp.w2))
    for t, (e, i) in enumerate(where):
        assert np.array_equal(out[e, i], y[t])
    for e in range(p.E):
        assert np.all(out[e, counts[e]:] == 0)


def test_batched_empty_expert_and_bad_count():
    p = synth.Problem(M=4, H=128, I=128, E=3, topk=1)
    inp = synth.make_inputs(p, "cpu")
    a = np.tile(bits16(inp.x)[:2][None], (3, 1, 1))
    out = oracle.batched_experts_bf16(a, np.array([2, 0, 1], np.int32), bits16(inp.w13), bits16(inp.w2))
    assert np.all(out[1] == 0) and np.all(out[2, 1] == 0) and np.any(out[0] != 0)
    with pytest.raises(ValueError):
        oracle.batched_experts_bf16(a, np.array([1, -1, 0], np.int32), bits16(inp.w13), bits16(inp.w2))
