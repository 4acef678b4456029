"""The path at the limits of the interface on the GPU: the largest expert count and
top-k (256 experts, top-32), a single expert, more rows than one grid dimension
holds, and no tokens at all through every entry point. Each against the oracle (bit
for bit for ids and layouts, within the layer tolerance for y) or, for the 8-bit
forms at 70000 tokens, against the float64 layer within the derived bound."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
import quant_bound as qb
from hostutil import bf16_f64, bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, check_align, log, oracle_layer, run_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


@pytest.mark.parametrize("E,k", [(256, 32), (256, 1), (32, 32), (1, 1)])
def test_router_at_the_limits(E, k):
    g = torch.Generator().manual_seed(E * 100 + k)
    logits = torch.randn(700, E, generator=g)
    logits[::7] = torch.round(logits[::7] * 4) / 4     # frequent exact ties
    ids, w = moe.moe_topk(logits.to(DEV), k)
    ids_ref, w_ref = oracle.topk(logits.numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6


@pytest.mark.parametrize("M,k,E,B", [(3000, 32, 256, 16), (3000, 32, 256, 128), (513, 32, 64, 256),
                                     (4000, 1, 1, 128)])
def test_align_at_the_limits(M, k, E, B):
    g = np.random.default_rng(M + k + E + B)
    ids = np.stack([g.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
    check_align(ids, E, B)


@pytest.mark.parametrize("cfg", [
    dict(M=40, H=256, I=256, E=256, topk=32, block_m=16),
    dict(M=40, H=256, I=256, E=256, topk=32, block_m=128),
    dict(M=40, H=256, I=256, E=256, topk=32, block_m=64, wdtype="fp8"),
    dict(M=300, H=384, I=256, E=1, topk=1, block_m=256),
    dict(M=300, H=384, I=256, E=1, topk=1, block_m=128, wdtype="fp8"),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_at_the_limits(cfg):
    p = synth.Problem(**cfg)
    log(f"limits {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_layer(p, d, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert_close(bits16(y), oracle_layer(p, inp, ids_ref, w_ref), TOL[p.wdtype], str(cfg))


@pytest.mark.parametrize("cfg", [
    dict(M=70000, H=128, I=128, E=4, topk=2, block_m=16),
    dict(M=70000, H=128, I=128, E=4, topk=2, block_m=64),
    dict(M=70000, H=128, I=128, E=4, topk=2, block_m=64, wdtype="fp8"),
    dict(M=70000, H=256, I=256, E=4, topk=1, block_m=128, wdtype="mxfp8"),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_with_more_rows_than_one_grid_dimension(cfg):
    # The per-row kernels put rows along the grid's y dimension, which holds at most
    # 65536 workgroups: here the tokens (activation quantisers, reduce) and the padded
    # rows (separate activation pass) exceed it, and every token is checked. bf16
    # against the oracle within the layer tolerance; the 8-bit forms against the
    # float64 layer within the derived bound (quant_bound.py), since over 9 million
    # outputs a few z codes that round the other way can move single outputs past
    # the 6e-2 rule, on either side's rounding
    p = synth.Problem(**cfg)
    log(f"rows beyond grid y {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    ids, w = torch.from_numpy(ids_ref).to(DEV), torch.from_numpy(w_ref).to(DEV)
    if p.wdtype == "bf16":
        y = run_layer(p, d, ids, w)
        torch.cuda.synchronize()
        assert_close(bits16(y), oracle_layer(p, inp, ids_ref, w_ref), TOL[p.wdtype], str(cfg))
        return
    if p.wdtype == "mxfp8":
        prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, moe.MOE_W_MXFP8)
        s13, s2 = moe.moe_pack_mx_scales(prob, 1, d.w13s), moe.moe_pack_mx_scales(prob, 2, d.w2s)
        y = moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, s13, s2)
        W13 = qb.deq_mx(bits8(inp.w13q), inp.w13s.numpy(), False)
        W2 = qb.deq_mx(bits8(inp.w2q), inp.w2s.numpy(), False)
        act = qb.MX_32
    else:
        y = run_layer(p, d, ids, w)
        W13 = qb.deq_fp8_block(bits8(inp.w13q), inp.w13s.numpy())
        W2 = qb.deq_fp8_block(bits8(inp.w2q), inp.w2s.numpy())
        act = qb.FP8_128
    torch.cuda.synchronize()
    ref, bound = qb.layer_reference(bf16_f64(bits16(inp.x)), ids_ref, w_ref, W13, W2, act, fp32_acc=True)
    qb.check(bf16_f64(bits16(y)), ref, bound, str(cfg))


def test_no_tokens_through_every_entry_point():
    E, k, H, I = 8, 2, 256, 256
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((0, E), dtype=torch.float32, device=DEV)
    ids, w = moe.moe_topk(logits, k)
    assert ids.shape == (0, k) and w.shape == (0, k)
    s, e, npp, inv = moe.moe_align_block_size(ids, E, 16)
    torch.cuda.synchronize()
    assert int(npp.item()) == 0
    w13 = torch.randn(E, 2 * I, H, device=DEV).to(torch.bfloat16)
    w2 = torch.randn(E, H, I, device=DEV).to(torch.bfloat16)
    for block_m in (16, 128):
        y = moe.fused_experts(x, w13, w2, ids, w, block_m)
        assert y.shape == (0, H)
    q, sc = moe.moe_quant_fp8_groups(x)
    assert q.shape == (0, H) and sc.shape == (0, H // 128)
    torch.cuda.synchronize()
