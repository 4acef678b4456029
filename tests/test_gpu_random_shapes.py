"""Seeded sweep of small random problems through fused_experts against the oracle.

Each case draws its own sizes (H, I multiples of 128; ragged M; E from 1 to 64;
top-k up to 8), block size, weight format and layout, routing-weight placement,
and sometimes an expert map (one rank of an expert-parallel split) or token
chunks, so that tile tails, empty experts, single-token blocks and every kernel
family meet inputs no hand-written case chose. The tolerance is the layer's
(2e-2 bf16, 6e-2 for the 8-bit formats, relative to max(1, |y|), each against the
oracle of its own format).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
from hostutil import bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log, to_dev

pytestmark = pytest.mark.gpu


def draw_case(i: int) -> dict:
    g = np.random.default_rng(1000 + i)
    u = g.random()
    wdtype = "bf16" if u < 0.55 else "fp8" if u < 0.8 else "mxfp8" if u < 0.9 else "w4a8"
    mx = wdtype in ("mxfp8", "w4a8")
    block_m = int(128 if mx else g.choice([32, 64, 128]) if wdtype == "fp8" else g.choice([16, 32, 64, 128, 256]))
    E = int(g.integers(1, 65))
    cfg = dict(M=int(g.integers(1, 301)), H=128 * int(g.integers(1, 9)), I=128 * int(g.integers(1, 9)),
               E=E, topk=int(g.integers(1, min(E, 8) + 1)), block_m=block_m, wdtype=wdtype,
               bias_std=float(g.choice([0.0, 1.5])), seed=int(g.integers(0, 1000)),
               apply_router_weight_on_input=bool(g.random() < 0.25))
    if wdtype != "bf16" and block_m == 128:
        cfg["H"], cfg["I"] = max(cfg["H"], 256), max(cfg["I"], 256)  # the persistent kernel's K >= 256
    r = g.random()
    if r < 0.2 and E >= 4 and not mx:
        ep_size = int(g.choice([s for s in (2, 4) if E % s == 0] or [1]))
        if ep_size > 1:
            cfg.update(ep_size=ep_size, ep_rank=int(g.integers(0, ep_size)))
    elif r < 0.3 and cfg["M"] > 20:
        cfg["chunk_tokens"] = int(g.integers(8, cfg["M"]))
    return cfg


CASES = [draw_case(i) for i in range(200)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


@pytest.mark.parametrize("cfg", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_random_problem_matches_oracle(cfg):
    p = synth.Problem(**cfg)
    log(f"random {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    emap = None if inp.expert_map is None else inp.expert_map.to(DEV)
    ids, w = moe.moe_topk(d.logits, p.topk)
    on = p.apply_router_weight_on_input
    tiled = p.wdtype == "bf16" and p.block_m in (16, 128, 256) and cfg["seed"] % 2 == 0
    if p.wdtype in ("mxfp8", "w4a8"):
        prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m,
                                moe.MOE_W_MXFP8 if p.wdtype == "mxfp8" else moe.MOE_W_W4A8_MXFP4)
        s13, s2 = moe.moe_pack_mx_scales(prob, 1, d.w13s), moe.moe_pack_mx_scales(prob, 2, d.w2s)
        y = moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, s13, s2, apply_router_weight_on_input=on,
                              chunk_tokens=p.chunk_tokens)
    elif p.wdtype == "fp8":
        y = moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, d.w13s, d.w2s, apply_router_weight_on_input=on,
                              expert_map=emap, chunk_tokens=p.chunk_tokens)
    else:
        w13, w2, layout = d.w13, d.w2, moe.MOE_LAYOUT_ROWS
        if tiled:
            # (the packing problem names the held experts only; top-k does not matter to it)
            prob = moe.make_problem(p.M, p.H, p.I, len(p.local_experts), 1, p.block_m)
            w13, w2 = moe.moe_pack_weights(prob, 1, w13), moe.moe_pack_weights(prob, 2, w2)
            layout = moe.MOE_LAYOUT_TILED
        y = moe.fused_experts(d.x, w13, w2, ids, w, p.block_m, apply_router_weight_on_input=on,
                              weight_layout=layout, expert_map=emap, chunk_tokens=p.chunk_tokens)
    torch.cuda.synchronize()
    # the oracle's own router: ids bit for bit, weights within 1e-6, and its weights feed
    # the oracle layer
    ids_np, w_np = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_np)
    assert np.abs(w.cpu().numpy() - w_np).max() <= 1e-6
    em = None if inp.expert_map is None else inp.expert_map.numpy()
    if p.wdtype in ("mxfp8", "w4a8"):
        y_ref = oracle.fused_experts_mx(bits16(inp.x), bits8(inp.w13q) if p.wdtype == "mxfp8" else inp.w13q.numpy(),
                                        inp.w13s.numpy(), bits8(inp.w2q) if p.wdtype == "mxfp8" else inp.w2q.numpy(),
                                        inp.w2s.numpy(), ids_np, w_np, w4=p.wdtype == "w4a8", on_input=on)
    elif p.wdtype == "fp8":
        y_ref = oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                         inp.w2s.numpy(), ids_np, w_np, on_input=on, expert_map=em)
    else:
        y_ref = oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13), bits16(inp.w2), ids_np, w_np,
                                          on_input=on, expert_map=em)
    assert_close(bits16(y), y_ref, TOL["bf16" if p.wdtype == "bf16" else "fp8"], str(cfg))
