"""The seeded input generator: determinism, independence, recipe."""
import math

import numpy as np
import pytest
import torch

import synth


def test_deterministic_and_seed_dependent():
    p = synth.Problem(M=16, H=128, I=128, E=4, topk=2)
    a, b = synth.make_inputs(p, "cpu"), synth.make_inputs(p, "cpu")
    assert torch.equal(a.x, b.x) and torch.equal(a.w13, b.w13) and torch.equal(a.logits, b.logits)
    c = synth.make_inputs(synth.Problem(M=16, H=128, I=128, E=4, topk=2, seed=1), "cpu")
    assert not torch.equal(a.x, c.x)
    # tensors and experts draw from distinct streams
    assert not torch.equal(a.x.float()[:, :4], a.logits[:, :4])
    assert not torch.equal(a.w13[0], a.w13[1])


def test_per_expert_streams_do_not_depend_on_expert_count():
    a = synth.make_inputs(synth.Problem(M=4, H=128, I=128, E=2, topk=1), "cpu")
    b = synth.make_inputs(synth.Problem(M=4, H=128, I=128, E=5, topk=1), "cpu")
    assert torch.equal(a.w13[1], b.w13[1]) and torch.equal(a.w2[0], b.w2[0])


def test_recipe_statistics():
    p = synth.Problem(M=512, H=1024, I=256, E=4, topk=2, bias_std=1.5)
    inp = synth.make_inputs(p, "cpu")
    assert inp.x.dtype == torch.bfloat16 and inp.logits.dtype == torch.float32
    assert abs(inp.x.float().std().item() - 1.0) < 0.02
    assert abs(inp.w13.float().std().item() - 1 / math.sqrt(1024)) < 0.02 / math.sqrt(1024)
    assert abs(inp.w2.float().std().item() - 1 / math.sqrt(256)) < 0.02 / math.sqrt(256)
    # the per-expert bias shifts whole columns of the logits
    col_means = inp.logits.mean(0)
    assert col_means.std().item() > 0.3


def test_fp8_block_quant_recipe():
    p = synth.Problem(M=2, H=256, I=128, E=2, topk=1, wdtype="fp8")
    inp = synth.make_inputs(p, "cpu")
    assert inp.w13q.dtype == torch.float8_e4m3fn and inp.w13s.shape == (2, 2, 2)
    assert inp.w2s.shape == (2, 2, 1)
    # every block's largest code is 448 and dequantised values stay within one
    # e4m3 half-ulp of the block amax
    q = inp.w13q.float().view(2, 2, 128, 2, 128)
    assert torch.all(q.abs().amax(dim=(2, 4)) == 448.0)


def test_expert_parallel_rank_holds_its_slice_of_the_same_weights():
    full = synth.make_inputs(synth.Problem(M=8, H=128, I=128, E=8, topk=2), "cpu")
    for wdtype in ("bf16", "fp8"):
        p = synth.Problem(M=8, H=128, I=128, E=8, topk=2, wdtype=wdtype, ep_size=4, ep_rank=2)
        r = synth.make_inputs(p, "cpu")
        assert list(p.local_experts) == [4, 5]
        assert r.expert_map.tolist() == [-1, -1, -1, -1, 0, 1, -1, -1]
        assert torch.equal(r.x, full.x) and torch.equal(r.logits, full.logits)  # global routing
        if wdtype == "bf16":
            assert torch.equal(r.w13, full.w13[4:6]) and torch.equal(r.w2, full.w2[4:6])
        else:
            assert r.w13q.shape[0] == 2 and r.w2s.shape[0] == 2
    assert synth.make_inputs(synth.Problem(M=2, H=128, I=128, E=4, topk=1), "cpu").expert_map is None


@pytest.mark.parametrize("wdtype", ["mxfp8", "w4a8"])
@pytest.mark.parametrize("stack", [1 << 27, 2 * 256 * 128 * 3])  # one stack; stacks of 3 experts
def test_mx_weights_are_each_experts_own_quantisation(monkeypatch, wdtype, stack):
    monkeypatch.setattr(synth, "_MX_STACK", stack)
    p = synth.Problem(M=4, H=128, I=256, E=7, topk=2, wdtype=wdtype, block_m=128)
    d = synth.make_inputs(p, "cpu")
    fmt = "e4m3" if wdtype == "mxfp8" else "e2m1"
    for e in range(p.E):
        m13 = synth._randn((2 * p.I, p.H), "cpu", p.seed, synth._T_W13, e, 1.0 / math.sqrt(p.H))
        q, s = synth.mx_quant(m13.to(torch.bfloat16), fmt)
        assert torch.equal(d.w13q[e].view(torch.uint8), q.view(torch.uint8)) and torch.equal(d.w13s[e], s)
        m2 = synth._randn((p.H, p.I), "cpu", p.seed, synth._T_W2, e, 1.0 / math.sqrt(p.I))
        q, s = synth.mx_quant(m2.to(torch.bfloat16), fmt)
        assert torch.equal(d.w2q[e].view(torch.uint8), q.view(torch.uint8)) and torch.equal(d.w2s[e], s)
