"""Tiled weights (16 x 32 tiles, bf16, block_m 16 / 128 / 256): moe_pack_weights
writes the documented permutation, and every path that reads tiled weights
gives the bits of the same path on row-major weights (the kernels load the
same values into the same registers and LDS slots in the same order), which
the oracle parity tests pin; small cases are also checked against the oracle
directly, and the full-size workloads bit for bit against row-major weights."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
from hostutil import bits16
from test_gpu_parity import DEV, TOL, assert_close, log, to_dev

pytestmark = pytest.mark.gpu
TILED = moe.MOE_LAYOUT_TILED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def tiled_reference(w: torch.Tensor) -> torch.Tensor:
    # tiled[e][n/16][k/32][n%16][k%32] = w[e][n][k]
    E, N, K = w.shape
    return w.view(E, N // 16, 16, K // 32, 32).permute(0, 1, 3, 2, 4).contiguous().view(E, N, K)


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
        assert torch.equal(wp.view(torch.int16), tiled_reference(w).view(torch.int16))


def test_pack_weights_rejects_overlap_and_fp8():
    w = torch.zeros((2, 256, 128), dtype=torch.bfloat16, device=DEV)
    prob = moe.make_problem(1, 128, 128, 2, 1, 16)
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(prob, 1, w, out=w)
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(moe.make_problem(1, 128, 128, 2, 1, 128, moe.MOE_W_FP8_E4M3_BLOCK128), 1, w)


TILED_CASES = [
    dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16),               # decode workload (ring depths 4 / 2)
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16),                  # tiny workload (depth 2)
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=16),                 # odd chunk counts (depth 1)
    dict(M=21, H=384, I=256, E=6, topk=3, block_m=16, apply_router_weight_on_input=True),
    dict(M=200, H=512, I=256, E=4, topk=2, block_m=16),                 # many blocks per expert
    dict(M=1, H=256, I=256, E=4, topk=2, block_m=16),                   # one token
    dict(M=150, H=512, I=384, E=7, topk=3, block_m=128),                # partial column tile, split-K tail
    dict(M=1, H=256, I=128, E=4, topk=2, block_m=128),                  # one token, one column tile
    dict(M=300, H=256, I=640, E=5, topk=2, block_m=256),                # 5 column tiles
    dict(M=90, H=384, I=256, E=4, topk=2, block_m=256, apply_router_weight_on_input=True),
    dict(M=600, H=640, I=384, E=3, topk=2, block_m=128),                # several blocks per expert
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


def tiled_weights(p, d):
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m)
    return moe.moe_pack_weights(prob, 1, d.w13), moe.moe_pack_weights(prob, 2, d.w2)


@pytest.mark.parametrize("cfg", TILED_CASES, ids=CASE_ID)
def test_layer_tiled_matches_rows_and_oracle(cfg):
    p = synth.Problem(**cfg)
    log(f"tiled layer {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    ids, w = moe.moe_topk(d.logits, p.topk)
    on, B = p.apply_router_weight_on_input, p.block_m
    y_rows = moe.fused_experts(d.x, d.w13, d.w2, ids, w, B, apply_router_weight_on_input=on)
    w13t, w2t = tiled_weights(p, d)
    y_tiled = moe.fused_experts(d.x, w13t, w2t, ids, w, B, apply_router_weight_on_input=on,
                                weight_layout=TILED)
    torch.cuda.synchronize()
    assert torch.equal(y_rows.view(torch.int16), y_tiled.view(torch.int16))
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y_ref = oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13), bits16(inp.w2), ids_ref, w_ref,
                                      on_input=on)
    assert_close(bits16(y_tiled), y_ref, TOL["bf16"], str(cfg))


@pytest.mark.parametrize("cfg", [TILED_CASES[i] for i in (0, 2, 3, 6, 8)], ids=CASE_ID)
def test_stages_tiled_match_rows(cfg):
    # GEMM1 (plain and with the SiLU epilogue) and GEMM2 (with and without its
    # split-K workspace), stage by stage
    p = synth.Problem(**cfg)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    on, B = p.apply_router_weight_on_input, p.block_m
    rows = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, B, on_input=on)
    tiled = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, B, on_input=on, weight_layout=TILED)
    w13t, w2t = tiled_weights(p, d)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, B)
    cap, n = s.numel(), int(npp.item())
    out = {}
    for name, prob, w13, w2 in (("rows", rows, d.w13, d.w2), ("tiled", tiled, w13t, w2t)):
        h = torch.zeros((cap, 2 * p.I), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 1, d.x, w13, s, e, npp, h)
        z = torch.zeros((cap, p.I), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm_act(prob, d.x, None, w13, None, s, e, npp, w, z)
        o1 = torch.zeros((cap, p.H), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 2, z, w2, None, e, npp, o1)
        o2 = torch.zeros((cap, p.H), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 2, z, w2, None, e, npp, o2, workspace=moe.gemm_workspace_for(prob, DEV))
        out[name] = (h[:n], z[:n], o1[:n], o2[:n])
    torch.cuda.synchronize()
    for a, b in zip(out["rows"], out["tiled"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name,block_m", [("decode_m32", None), ("mixtral_prefill_m4096", None),
                                          ("mixtral_prefill_m4096", 256),
                                          ("dsv3_skewed_prefill_m8192", None)])
def test_full_size_tiled_matches_rows(name, block_m):
    # the launch configuration bench.py times (and the Mixtral shape in 256-row
    # blocks); row-major results are checked against the oracle on sampled tokens
    # by the parity tests
    p = synth.Problem.named(name, **({} if block_m is None else {"block_m": block_m}))
    log(f"full-size tiled {name} block_m {p.block_m}")
    d = synth.make_inputs(p, DEV)
    ids, w = moe.moe_topk(d.logits, p.topk)
    y_rows = moe.fused_experts(d.x, d.w13, d.w2, ids, w, p.block_m)
    w13t, w2t = tiled_weights(p, d)
    del d.w13, d.w2
    y_tiled = moe.fused_experts(d.x, w13t, w2t, ids, w, p.block_m, weight_layout=TILED)
    torch.cuda.synchronize()
    assert torch.equal(y_rows.view(torch.int16), y_tiled.view(torch.int16))


def test_tiled_layout_unsupported_block_sizes():
    p = synth.Problem(M=64, H=256, I=256, E=4, topk=2, block_m=64)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    with pytest.raises(moe.MoeError) as err:
        moe.fused_experts(d.x, d.w13, d.w2, ids, w, 64, weight_layout=TILED)
    assert err.value.status == moe.MOE_E_UNSUPPORTED
