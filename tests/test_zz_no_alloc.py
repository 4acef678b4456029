"""fused_experts_static (the entry point that allocates nothing) against fused_experts.

Each case makes two calls in a row through the C ABI, the second with fewer
tokens, both into the same static scratch, and compares each with fused_experts
on a caller workspace: bit for bit where the two run the same kernels (no
split-K tail in the second GEMM), else within the layer tolerance. A problem
whose scratch exceeds the static array is refused with MOE_E_WORKSPACE.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import synth
from hostutil import bits16
from test_gpu_parity import DEV, TOL, assert_close, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


CASES = [
    # (problem, smaller token count of the second call, weight layout)
    (dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16), 5, moe.MOE_LAYOUT_TILED),   # decode workload
    (dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16), 7, moe.MOE_LAYOUT_ROWS),
    (dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"), 40, moe.MOE_LAYOUT_ROWS),
    (dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8", apply_router_weight_on_input=True), 9,
     moe.MOE_LAYOUT_ROWS),
    (dict(M=300, H=512, I=384, E=5, topk=2, block_m=128), 64, moe.MOE_LAYOUT_TILED),
    (dict(M=300, H=512, I=384, E=3, topk=2, block_m=256), 100, moe.MOE_LAYOUT_ROWS),
    (dict(M=1000, H=256, I=256, E=8, topk=2, block_m=64, chunk_tokens=256), 300, moe.MOE_LAYOUT_ROWS),
    (dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="mxfp8"), 33, moe.MOE_LAYOUT_ROWS),
]


def weights(p, d, layout):
    if p.wdtype == "bf16":
        w13, w2 = d.w13, d.w2
        if layout == moe.MOE_LAYOUT_TILED:
            rows = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m)
            w13, w2 = moe.moe_pack_weights(rows, 1, w13), moe.moe_pack_weights(rows, 2, w2)
        return w13, w2, None, None
    s13, s2 = d.w13s, d.w2s
    if p.wdtype == "mxfp8":
        prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, moe.MOE_W_MXFP8)
        s13, s2 = moe.moe_pack_mx_scales(prob, 1, s13), moe.moe_pack_mx_scales(prob, 2, s2)
    return d.w13q, d.w2q, s13, s2


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c[0].items()) + f"-then{c[1]}")
def test_static_scratch_matches_fused_experts(case):
    cfg, m2, layout = case
    p = synth.Problem(**cfg)
    log(f"static scratch {cfg}, then M={m2}")
    d = to_dev(synth.make_inputs(p, "cpu"))
    w13, w2, s13, s2 = weights(p, d, layout)
    ids, w = moe.moe_topk(d.logits, p.topk)
    on = p.apply_router_weight_on_input
    split = p.wdtype == "bf16" and p.block_m in (128, 256)   # fused_experts' split-K tail
    for M in (p.M, m2):                                      # two calls, the second smaller
        x, i, ww = d.x[:M].contiguous(), ids[:M].contiguous(), w[:M].contiguous()
        y_ref = moe.fused_experts(x, w13, w2, i, ww, p.block_m, s13, s2, apply_router_weight_on_input=on,
                                  weight_layout=layout, chunk_tokens=p.chunk_tokens)
        y = torch.full_like(x, float("nan"))
        moe.fused_experts_static(x, w13, w2, i, ww, p.block_m, y, s13, s2, apply_router_weight_on_input=on,
                                 weight_layout=layout, chunk_tokens=p.chunk_tokens)
        torch.cuda.synchronize()
        if split:
            assert_close(bits16(y), bits16(y_ref), TOL[p.wdtype if p.wdtype == "bf16" else "fp8"], f"M={M}")
        else:
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"M={M}: bits differ"


def test_static_scratch_refuses_a_problem_beyond_its_size():
    p = synth.Problem(M=4096, H=2048, I=2048, E=8, topk=2, block_m=128)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = torch.empty_like(d.x)
    with pytest.raises(moe.MoeError) as ei:
        moe.fused_experts_static(d.x, d.w13, d.w2, ids, w, p.block_m, y)
    assert ei.value.status == moe.MOE_E_WORKSPACE
    # the same problem in chunks of 512 tokens fits, and matches fused_experts
    moe.fused_experts_static(d.x, d.w13, d.w2, ids, w, p.block_m, y, chunk_tokens=512)
    y_ref = moe.fused_experts(d.x, d.w13, d.w2, ids, w, p.block_m, chunk_tokens=512)
    torch.cuda.synchronize()
    assert_close(bits16(y), bits16(y_ref), TOL["bf16"], "chunked static")
    assert np.isfinite(y.float().cpu().numpy()).all()
