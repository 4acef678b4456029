"""MXFP8 (E4M3 with an E8M0 scale per 32 values) on the GPU: the activation
quantiser and the scale packing bit for bit, and the layer element by element
against the oracle (tolerance 6e-2 as for fp8), at small sizes and at full
size on sampled tokens."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import sampled
import synth
from hostutil import bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def test_quant_mx_bit_exact():
    g = torch.Generator().manual_seed(9)
    x = torch.randn(300, 7168, generator=g) * torch.exp2(torch.randint(-12, 12, (300, 1), generator=g))
    x[3, 64:96] = 0.0
    x[4, :32] = 448.0 * 2.0 ** -3      # amax exactly on a power-of-two boundary
    x[5, 32:64] = -1e-30
    xb = x.to(torch.bfloat16)
    q, s = moe.moe_quant_mx_groups(xb.to(DEV))
    q_ref, s_ref = oracle.quant_mx_fp8(xb.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(bits8(q), q_ref)


def test_pack_mx_scales_is_the_documented_order():
    E, I, H = 3, 256, 512
    prob = moe.make_problem(1, H, I, E, 1, 128, moe.MOE_W_MXFP8)
    g = torch.Generator().manual_seed(2)
    for which, (N, K) in ((1, (2 * I, H)), (2, (H, I))):
        s = torch.randint(0, 255, (E, N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
        packed = moe.moe_pack_mx_scales(prob, which, s.to(DEV)).cpu()
        ref = s.view(E, N, K // 128, 4).permute(0, 2, 1, 3).contiguous().view(torch.int32).view(E, K // 128, N)
        assert torch.equal(packed, ref)


def mx_weights(p, d):
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, moe.MOE_W_MXFP8)
    return moe.moe_pack_mx_scales(prob, 1, d.w13s), moe.moe_pack_mx_scales(prob, 2, d.w2s)


def run_mx(p, d, ids, w):
    s13, s2 = mx_weights(p, d)
    return moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, s13, s2,
                             apply_router_weight_on_input=p.apply_router_weight_on_input)


def oracle_mx(p, inp, ids, w, toks=None):
    x = bits16(inp.x) if toks is None else bits16(inp.x[toks])
    return oracle.fused_experts_mx(x, bits8(inp.w13q), inp.w13s.cpu().numpy(), bits8(inp.w2q),
                                   inp.w2s.cpu().numpy(), ids, w, on_input=p.apply_router_weight_on_input)


CASES = [
    dict(M=150, H=512, I=256, E=7, topk=3),
    dict(M=200, H=384, I=640, E=6, topk=2),                                  # ragged GEMM2 tile, 5 z blocks
    dict(M=300, H=256, I=256, E=4, topk=2, apply_router_weight_on_input=True),
    dict(M=1, H=512, I=256, E=4, topk=2),
    dict(M=64, H=1024, I=512, E=16, topk=4),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_mx_matches_oracle(cfg):
    p = synth.Problem(**cfg, wdtype="mxfp8", block_m=128)
    log(f"mx layer {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = synth.Inputs(*[None if t is None else t.to(DEV) for t in (
        inp.x, inp.logits, inp.w13, inp.w2, inp.w13q, inp.w13s, inp.w2q, inp.w2s)])
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_mx(p, d, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y_ref = oracle_mx(p, inp, ids_ref, w_ref)
    assert_close(bits16(y), y_ref, TOL["fp8"], str(cfg))


def full_size_mx_sampled(name, run):
    p = synth.Problem.named(name)
    w4 = p.wdtype == "w4a8"
    log(f"full-size {name}")
    d = synth.make_inputs(p, DEV)
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run(p, d, ids, w)
    torch.cuda.synchronize()
    ids_np, w_np = oracle.topk(d.logits.cpu().numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_np)
    toks = sampled.pick_tokens(ids_np, p.E, p.block_m)
    experts, sub_ids = sampled.expert_subset(ids_np, toks, p.E)
    sel = torch.tensor(experts, device=DEV)
    log(f"full-size {name}: oracle on {len(toks)} tokens ({len(experts)} experts)")
    y_ref = oracle.fused_experts_mx(bits16(d.x[toks]), bits8(d.w13q[sel]), d.w13s[sel].cpu().numpy(),
                                    bits8(d.w2q[sel]), d.w2s[sel].cpu().numpy(), sub_ids, w_np[toks], w4=w4)
    assert_close(bits16(y[toks]), y_ref, TOL["fp8"], name)
    assert bool(torch.isfinite(y.float()).all())


def test_full_size_mx_sampled():
    full_size_mx_sampled("mxfp8_m4096", run_mx)


# ------------------------------------------------------------------- W4A8 ---

def run_w4(p, d, ids, w):
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, moe.MOE_W_W4A8_MXFP4)
    s13, s2 = moe.moe_pack_mx_scales(prob, 1, d.w13s), moe.moe_pack_mx_scales(prob, 2, d.w2s)
    return moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, s13, s2,
                             apply_router_weight_on_input=p.apply_router_weight_on_input)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_w4a8_matches_oracle(cfg):
    p = synth.Problem(**cfg, wdtype="w4a8", block_m=128)
    log(f"w4a8 layer {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = synth.Inputs(*[None if t is None else t.to(DEV) for t in (
        inp.x, inp.logits, inp.w13, inp.w2, inp.w13q, inp.w13s, inp.w2q, inp.w2s)])
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_w4(p, d, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y_ref = oracle.fused_experts_mx(bits16(inp.x), inp.w13q.numpy(), inp.w13s.numpy(), inp.w2q.numpy(),
                                    inp.w2s.numpy(), ids_ref, w_ref, w4=True,
                                    on_input=p.apply_router_weight_on_input)
    assert_close(bits16(y), y_ref, TOL["fp8"], str(cfg))


def test_full_size_w4a8_sampled():
    full_size_mx_sampled("w4a8_m4096", run_w4)
