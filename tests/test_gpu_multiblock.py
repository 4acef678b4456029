"""Experts of several 128-row blocks in the fp8-family layers.

With fp8 block-scaled, MXFP8 or W4A8 weights (block_m 128), the persistent GEMM
kernels walk tiles of many blocks per expert, sharing each expert's weight tiles
between its blocks through L2. fused_experts must give the bits of the stage entry
points launched one by one, and match the oracle, on routings that give experts one
to many blocks, a hot expert among cold ones, router weights on the input, and an
expert-parallel rank.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
from hostutil import bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


WDT = {"fp8": moe.MOE_W_FP8_E4M3_BLOCK128, "mxfp8": moe.MOE_W_MXFP8, "w4a8": moe.MOE_W_W4A8_MXFP4}

CASES = [
    # M, H, I, E, topk, wdtype, on_input, hot (logit bias on expert 0)
    (700, 256, 256, 5, 2, "fp8", False, 0.0),       # ~3 blocks per expert
    (1000, 256, 384, 4, 2, "fp8", False, 0.0),      # ~4 blocks
    (1200, 384, 256, 3, 2, "fp8", False, 0.0),      # ~7 blocks
    (1500, 256, 256, 16, 2, "fp8", False, 4.0),     # one hot expert with many blocks, cold ones with one
    (640, 512, 256, 8, 2, "fp8", True, 0.0),        # router weight on the input
    (900, 256, 256, 6, 3, "w4a8", False, 0.0),
    (1500, 256, 384, 16, 2, "w4a8", False, 4.0),
    (1000, 256, 256, 4, 2, "mxfp8", False, 0.0),
    (1500, 384, 256, 16, 2, "mxfp8", True, 4.0),
]
CASE_ID = lambda c: f"M{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}-k{c[4]}-{c[5]}" + ("-oninput" if c[6] else "") + \
    (f"-hot{c[7]:g}" if c[7] else "")


def weights_and_scales(p, d):
    if p.wdtype in ("mxfp8", "w4a8"):
        prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, WDT[p.wdtype])
        return d.w13q, moe.moe_pack_mx_scales(prob, 1, d.w13s), d.w2q, moe.moe_pack_mx_scales(prob, 2, d.w2s)
    return d.w13q, d.w13s, d.w2q, d.w2s


def staged(p, d, ids, w, w13, s13, w2, s2):
    """The layer through the stage entry points."""
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, WDT[p.wdtype], p.apply_router_weight_on_input)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, p.block_m)
    cap = s.numel()
    mx = p.wdtype == "mxfp8"  # E8M0 activation scales, four to an int32 word
    sdt = torch.int32 if mx else torch.float32
    if mx:
        xq, xs = moe.moe_quant_mx_groups(d.x)
        xs = xs.view(torch.int32)
    else:
        xq, xs = moe.moe_quant_fp8_groups(d.x)
    xst = torch.empty((p.H // 128, cap), dtype=sdt, device=DEV)
    moe.moe_permute_scales(prob, xs, s, npp, xst)
    z = torch.empty((cap, p.I), dtype=torch.float8_e4m3fn, device=DEV)
    zs = torch.empty((p.I // 128, cap), dtype=sdt, device=DEV)
    moe.moe_expert_gemm_act(prob, xq, xst, w13, s13, s, e, npp, w, z, zs)
    o = torch.empty((cap, p.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_expert_gemm(prob, 2, z, w2, None, e, npp, o, zs, s2)
    y = torch.empty_like(d.x)
    moe.moe_unpermute_reduce(prob, o, inv, w, y)
    return y, e, npp


@pytest.mark.parametrize("case", CASES, ids=CASE_ID)
def test_multiblock_layer_matches_the_stages_and_the_oracle(case):
    M, H, I, E, k, wdt, on_input, hot = case
    log(f"multi-block {CASE_ID(case)}")
    p = synth.Problem(M=M, H=H, I=I, E=E, topk=k, block_m=128, wdtype=wdt, apply_router_weight_on_input=on_input)
    inp = synth.make_inputs(p, "cpu")
    logits = inp.logits.clone()
    logits[:, 0] += hot
    d = synth.Inputs(*[None if t is None else t.to(DEV) for t in (
        inp.x, logits, inp.w13, inp.w2, inp.w13q, inp.w13s, inp.w2q, inp.w2s)])
    ids, w = moe.moe_topk(d.logits, k)
    w13, s13, w2, s2 = weights_and_scales(p, d)
    y = moe.fused_experts(d.x, w13, w2, ids, w, 128, s13, s2, apply_router_weight_on_input=on_input)
    y_st, e, npp = staged(p, d, ids, w, w13, s13, w2, s2)
    torch.cuda.synchronize()
    # the routing has experts of two or more blocks
    blocks = np.bincount(e.cpu().numpy()[: int(npp.item()) // 128], minlength=E)
    assert blocks.max() >= 2, blocks
    assert torch.equal(y.view(torch.int16), y_st.view(torch.int16)), "fused layer and stages differ"
    ids_ref, w_ref = oracle.topk(logits.numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    if wdt in ("mxfp8", "w4a8"):
        y_ref = oracle.fused_experts_mx(bits16(inp.x), bits8(inp.w13q) if wdt == "mxfp8" else inp.w13q.numpy(),
                                        inp.w13s.numpy(), bits8(inp.w2q) if wdt == "mxfp8" else inp.w2q.numpy(),
                                        inp.w2s.numpy(), ids_ref, w_ref, w4=wdt == "w4a8", on_input=on_input)
    else:
        y_ref = oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                         inp.w2s.numpy(), ids_ref, w_ref, on_input=on_input)
    assert_close(bits16(y), y_ref, TOL["fp8"], CASE_ID(case))


def test_multiblock_layer_on_an_expert_parallel_rank():
    # global routing over 16 experts, this rank holding 4 of them, each with
    # several blocks of local items
    p = synth.Problem(M=1200, H=256, I=256, E=16, topk=2, block_m=128, wdtype="fp8", ep_size=4, ep_rank=1)
    log("multi-block expert-parallel rank")
    inp = synth.make_inputs(p, "cpu")
    d = synth.Inputs(*[None if t is None else t.to(DEV) for t in (
        inp.x, inp.logits, inp.w13, inp.w2, inp.w13q, inp.w13s, inp.w2q, inp.w2s)])
    emap = inp.expert_map.to(DEV)
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, 128, d.w13s, d.w2s, expert_map=emap)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    y_ref = oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                     inp.w2s.numpy(), ids_ref, w_ref, expert_map=inp.expert_map.numpy())
    assert_close(bits16(y), y_ref, TOL["fp8"], "ep rank")
    # the rank's local routing has experts of several blocks
    s, e, npp, inv = moe.moe_align_block_size_ep(ids, emap, len(p.local_experts), 128)
    blocks = np.bincount(e.cpu().numpy()[: int(npp.item()) // 128], minlength=len(p.local_experts))
    assert blocks.max() >= 2, blocks
