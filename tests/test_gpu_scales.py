"""The 8-bit paths on inputs whose quantisation scales are spread over many powers of two.

With the pages' weight recipe (N(0, 1/sqrt(fan_in)) masters) every 128x128 block
has about the same amax, so a kernel that reads a neighbouring block's, group's
or expert's scale errs by a few percent and passes the layer tolerance. Here the
masters are multiplied by powers of two per block and per activation group
before quantisation (synth's scale_spread), so such a mistake moves outputs by
large factors. Each case is checked twice:

* signed inputs against the float64 layer on the dequantised weights, within the
  derived per-element bound of quant_bound.py (fp32 accumulation). Where the
  sums cancel, this bound is loose; it is also the right yardstick here, since
  an output's quantisation error scales with the largest terms of its row, not
  with the (cancelled) output itself: the oracle and the kernels each stay
  within it but may differ from each other by more than 6e-2 of a small output;
* the same inputs with the sign bits of x and of the weight codes cleared: with
  no cancellation the derived bound is a few percent of each value, and the
  outputs also agree with the oracle within the layer tolerance (6e-2 of
  max(1, |y|)).

Formats: fp8 128x128 blocks (block_m 32, 64 and the persistent 128 kernel, on-input
weights, an expert-parallel map, token chunks), MXFP8, W4A8, and the batched form.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
import quant_bound as qb
from hostutil import bf16_f64, bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def nonneg(inp: synth.Inputs, fp4: bool) -> synth.Inputs:
    """The same inputs with every sign bit of x and of the weight codes cleared."""
    x = (inp.x.view(torch.int16) & 0x7FFF).view(torch.bfloat16)
    m = 0x77 if fp4 else 0x7F
    q = lambda t: (t.view(torch.uint8) & m).view(t.dtype)
    return synth.Inputs(x, inp.logits, None, None, q(inp.w13q), inp.w13s, q(inp.w2q), inp.w2s,
                        expert_map=inp.expert_map)


def run_gpu(p: synth.Problem, inp: synth.Inputs, ids_np, w_np):
    dev = lambda t: None if t is None else t.to(DEV)
    ids, w = torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV)
    on = p.apply_router_weight_on_input
    emap = dev(inp.expert_map)
    if p.wdtype in ("mxfp8", "w4a8"):
        prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m,
                                moe.MOE_W_MXFP8 if p.wdtype == "mxfp8" else moe.MOE_W_W4A8_MXFP4)
        s13, s2 = moe.moe_pack_mx_scales(prob, 1, dev(inp.w13s)), moe.moe_pack_mx_scales(prob, 2, dev(inp.w2s))
    else:
        s13, s2 = dev(inp.w13s), dev(inp.w2s)
    y = moe.fused_experts(dev(inp.x), dev(inp.w13q), dev(inp.w2q), ids, w, p.block_m, s13, s2,
                          apply_router_weight_on_input=on, expert_map=emap, chunk_tokens=p.chunk_tokens)
    torch.cuda.synchronize()
    return bits16(y)


def run_oracle(p: synth.Problem, inp: synth.Inputs, ids_np, w_np):
    on = p.apply_router_weight_on_input
    if p.wdtype in ("mxfp8", "w4a8"):
        return oracle.fused_experts_mx(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                       inp.w2s.numpy(), ids_np, w_np, w4=p.wdtype == "w4a8", on_input=on)
    em = None if inp.expert_map is None else inp.expert_map.numpy()
    return oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                    inp.w2s.numpy(), ids_np, w_np, on_input=on, expert_map=em)


def exact_reference(p: synth.Problem, inp: synth.Inputs, ids_np, w_np):
    w4 = p.wdtype == "w4a8"
    if p.wdtype in ("mxfp8", "w4a8"):
        W13 = qb.deq_mx(bits8(inp.w13q), inp.w13s.numpy(), w4)
        W2 = qb.deq_mx(bits8(inp.w2q), inp.w2s.numpy(), w4)
    else:
        W13 = qb.deq_fp8_block(bits8(inp.w13q), inp.w13s.numpy())
        W2 = qb.deq_fp8_block(bits8(inp.w2q), inp.w2s.numpy())
    act = qb.MX_32 if p.wdtype == "mxfp8" else qb.FP8_128
    em = None if inp.expert_map is None else inp.expert_map.numpy()
    return qb.layer_reference(bf16_f64(bits16(inp.x)), ids_np, w_np, W13, W2, act,
                              p.apply_router_weight_on_input, fp32_acc=True, expert_map=em)


CASES = [
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=32, wdtype="fp8"),
    dict(M=40, H=384, I=256, E=5, topk=2, block_m=64, wdtype="fp8", apply_router_weight_on_input=True),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=200, H=384, I=640, E=6, topk=2, block_m=128, wdtype="fp8", apply_router_weight_on_input=True),
    dict(M=700, H=512, I=256, E=4, topk=2, block_m=128, wdtype="fp8"),      # persistent walk of many tiles
    dict(M=96, H=256, I=256, E=8, topk=2, block_m=128, wdtype="fp8", ep_size=2, ep_rank=1),
    dict(M=300, H=256, I=256, E=6, topk=2, block_m=128, wdtype="fp8", chunk_tokens=128),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="mxfp8"),
    dict(M=200, H=384, I=640, E=6, topk=2, block_m=128, wdtype="mxfp8", apply_router_weight_on_input=True),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="w4a8"),
    dict(M=200, H=256, I=384, E=6, topk=2, block_m=128, wdtype="w4a8", apply_router_weight_on_input=True),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


@pytest.mark.parametrize("cfg", CASES, ids=CASE_ID)
def test_spread_scales_layer(cfg):
    p = synth.Problem(**cfg, scale_spread=4, seed=31)
    log(f"spread scales {cfg}")
    inp = synth.make_inputs(p, "cpu")
    ids_np, w_np = oracle.topk(inp.logits.numpy(), p.topk)
    # signed inputs: the derived bound against the exact layer
    y = run_gpu(p, inp, ids_np, w_np)
    ref, bound = exact_reference(p, inp, ids_np, w_np)
    qb.check(bf16_f64(y), ref, bound, f"{cfg} (signed) vs the exact layer")
    # sign bits cleared: the (tight) derived bound, and the layer tolerance against the oracle
    pos = nonneg(inp, p.wdtype == "w4a8")
    y = run_gpu(p, pos, ids_np, w_np)
    ref, bound = exact_reference(p, pos, ids_np, w_np)
    worst = qb.check(bf16_f64(y), ref, bound, f"{cfg} vs the exact layer")
    assert_close(y, run_oracle(p, pos, ids_np, w_np), TOL["fp8"], f"{cfg} (non-negative) vs oracle")
    log(f"  worst err / bound {worst:.3f}")


def test_spread_scales_batched_fp8():
    p = synth.Problem(M=6 * 128, H=256, I=256, E=6, topk=1, block_m=128, wdtype="fp8", scale_spread=4, seed=32)
    inp = synth.make_inputs(p, "cpu")
    max_M = 128
    counts = np.array([128, 0, 77, 200, 1, 64], np.int32)
    for positive in (False, True):
        src = nonneg(inp, False) if positive else inp
        a = src.x.view(p.E, max_M, p.H)
        out = moe.moe_batched_experts(a.to(DEV), torch.from_numpy(counts).to(DEV), src.w13q.to(DEV),
                                      src.w2q.to(DEV), p.block_m, src.w13s.to(DEV), src.w2s.to(DEV))
        torch.cuda.synchronize()
        W13 = qb.deq_fp8_block(bits8(src.w13q), src.w13s.numpy())
        W2 = qb.deq_fp8_block(bits8(src.w2q), src.w2s.numpy())
        exact, bound = qb.batched_reference(bf16_f64(bits16(a)), counts, W13, W2, qb.FP8_128, fp32_acc=True)
        qb.check(bf16_f64(bits16(out)), exact, bound, f"batched fp8 (non-negative {positive}) vs the exact layer")
        if positive:
            ref = oracle.batched_experts_fp8(bits16(a), counts, bits8(src.w13q), src.w13s.numpy(),
                                             bits8(src.w2q), src.w2s.numpy())
            assert_close(bits16(out), ref, TOL["fp8"], "batched fp8 (non-negative) vs oracle")
