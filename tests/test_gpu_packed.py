"""The MFMA16 weight order (block_m 16, bf16): moe_pack_weights writes the
documented permutation, and every path that reads packed weights gives the
bits of the same path on row-major weights (both read the same values into
the same registers in the same order), which the oracle parity tests pin."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
from hostutil import bits16
from test_gpu_parity import DEV, TOL, assert_close, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def packed_reference(w: torch.Tensor) -> torch.Tensor:
    # packed[e][n/16][k/32][(k%32)/8][n%16][k%8] = w[e][n][k]
    E, N, K = w.shape
    return w.view(E, N // 16, 16, K // 32, 4, 8).permute(0, 1, 3, 4, 2, 5).contiguous().view(E, N, K)


@pytest.mark.parametrize("shape", [(3, 256, 128), (2, 512, 640), (128, 1536, 2048), (5, 256, 384)])
def test_pack_weights_is_the_documented_permutation(shape):
    E, N, K = shape
    log(f"pack {shape}")
    g = torch.Generator(device=DEV).manual_seed(11)
    w = torch.randint(-32768, 32767, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.int16)
    w = w.view(torch.bfloat16)
    # which = 1 packs w13 [E, 2I, H]; which = 2 packs w2 [E, H, I]
    p1 = moe.make_problem(1, K, N // 2, E, 1, 16)
    p2 = moe.make_problem(1, N, K, E, 1, 16)
    for prob, which in ((p1, 1), (p2, 2)):
        wp = moe.moe_pack_weights(prob, which, w)
        torch.cuda.synchronize()
        assert torch.equal(wp.view(torch.int16), packed_reference(w).view(torch.int16))


def test_pack_weights_rejects_overlap_and_fp8():
    w = torch.zeros((2, 256, 128), dtype=torch.bfloat16, device=DEV)
    prob = moe.make_problem(1, 128, 128, 2, 1, 16)
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(prob, 1, w, out=w)
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(moe.make_problem(1, 128, 128, 2, 1, 128, moe.MOE_W_FP8_E4M3_BLOCK128), 1, w)


PACKED_CASES = [
    dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16),               # decode workload (ring depths 4 / 2)
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16),                  # tiny workload (depth 2)
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=16),                 # odd chunk counts (depth 1)
    dict(M=21, H=384, I=256, E=6, topk=3, block_m=16, apply_router_weight_on_input=True),
    dict(M=200, H=512, I=256, E=4, topk=2, block_m=16),                 # many blocks per expert
    dict(M=1, H=256, I=256, E=4, topk=2, block_m=16),                   # one token
]


def packed_inputs(p, d):
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m)
    return moe.moe_pack_weights(prob, 1, d.w13), moe.moe_pack_weights(prob, 2, d.w2)


@pytest.mark.parametrize("cfg", PACKED_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_packed_matches_rows_and_oracle(cfg):
    p = synth.Problem(**cfg)
    log(f"packed layer {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    ids, w = moe.moe_topk(d.logits, p.topk)
    on = p.apply_router_weight_on_input
    y_rows = moe.fused_experts(d.x, d.w13, d.w2, ids, w, 16, apply_router_weight_on_input=on)
    w13p, w2p = packed_inputs(p, d)
    y_packed = moe.fused_experts(d.x, w13p, w2p, ids, w, 16, apply_router_weight_on_input=on,
                                 weight_layout=moe.MOE_LAYOUT_MFMA16)
    torch.cuda.synchronize()
    assert torch.equal(y_rows.view(torch.int16), y_packed.view(torch.int16))
    y_ref = oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13), bits16(inp.w2),
                                      ids.cpu().numpy(), w.cpu().numpy(), on_input=on)
    assert_close(bits16(y_packed), y_ref, TOL["bf16"], str(cfg))


@pytest.mark.parametrize("cfg", PACKED_CASES[:4], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_stages_packed_match_rows(cfg):
    # GEMM1 (plain and with the SiLU epilogue) and GEMM2, stage by stage
    p = synth.Problem(**cfg)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    on = p.apply_router_weight_on_input
    rows = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, 16, on_input=on)
    packed = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, 16, on_input=on,
                              weight_layout=moe.MOE_LAYOUT_MFMA16)
    w13p, w2p = packed_inputs(p, d)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, 16)
    cap, n = s.numel(), int(npp.item())
    out = {}
    for name, prob, w13, w2 in (("rows", rows, d.w13, d.w2), ("packed", packed, w13p, w2p)):
        h = torch.zeros((cap, 2 * p.I), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 1, d.x, w13, s, e, npp, h)
        z = torch.zeros((cap, p.I), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm_act(prob, d.x, None, w13, None, s, e, npp, w, z)
        o = torch.zeros((cap, p.H), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 2, z, w2, None, e, npp, o)
        out[name] = (h[:n], z[:n], o[:n])
    torch.cuda.synchronize()
    for a, b in zip(out["rows"], out["packed"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_packed_layout_unsupported_outside_block16():
    p = synth.Problem(M=64, H=256, I=256, E=4, topk=2, block_m=128)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    with pytest.raises(moe.MoeError) as err:
        moe.fused_experts(d.x, d.w13, d.w2, ids, w, 128, weight_layout=moe.MOE_LAYOUT_MFMA16)
    assert err.value.status == moe.MOE_E_UNSUPPORTED
