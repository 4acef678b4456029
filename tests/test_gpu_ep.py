"""Expert-parallel shard on one GPU (expert map with -1 for remote experts):
align is bit-exact with the oracle, the layer matches the oracle element by
element on every GEMM path, the ranks' outputs add up to the unsharded layer,
and the full-size rank of the skewed workload matches on sampled tokens."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import sampled
import synth
from hostutil import bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def random_map(g, E_global, E_local):
    emap = np.full(E_global, -1, np.int32)
    emap[g.choice(E_global, E_local, replace=False)] = g.permutation(E_local)
    return emap


def check_align_ep(ids_np, emap, E_local, B):
    s, x, npp, inv = moe.moe_align_block_size_ep(torch.from_numpy(ids_np).to(DEV),
                                                 torch.from_numpy(emap).to(DEV), E_local, B)
    rs, rx, rnpp, rinv = oracle.align(ids_np, E_local, B, expert_map=emap)
    assert int(npp.item()) == rnpp
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(x.cpu().numpy(), rx)
    assert np.array_equal(inv.cpu().numpy(), rinv)


def test_align_ep_bit_exact():
    g = np.random.default_rng(4)
    for M, k, Eg, El, B in [(64, 2, 8, 3, 16), (32, 8, 128, 16, 16), (3000, 8, 256, 32, 128),
                            (1, 2, 8, 4, 64), (500, 4, 16, 16, 256), (200, 2, 64, 1, 32)]:
        ids = np.stack([g.choice(Eg, k, replace=False) for _ in range(M)]).astype(np.int32)
        check_align_ep(ids, random_map(g, Eg, El), El, B)
    ids = np.stack([g.choice(16, 4, replace=False) for _ in range(100)]).astype(np.int32)
    check_align_ep(ids, np.full(16, -1, np.int32), 4, 16)                       # nothing local
    check_align_ep(ids, np.arange(16, dtype=np.int32), 16, 16)                  # identity
    check_align_ep(ids, np.where(np.arange(16) < 8, np.arange(16), 99).astype(np.int32), 8, 16)


EP_CASES = [
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16, ep_size=4, ep_rank=1),
    dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16, ep_size=8, ep_rank=3),     # decode shard
    dict(M=130, H=640, I=384, E=16, topk=4, block_m=128, ep_size=2, ep_rank=0),
    dict(M=300, H=512, I=384, E=12, topk=2, block_m=256, ep_size=3, ep_rank=2),
    dict(M=37, H=384, I=256, E=12, topk=3, block_m=32, ep_size=4, ep_rank=0),
    dict(M=64, H=256, I=512, E=16, topk=4, block_m=64, ep_size=8, ep_rank=7,
         apply_router_weight_on_input=True),
    dict(M=150, H=512, I=256, E=14, topk=3, block_m=128, wdtype="fp8", ep_size=2, ep_rank=1),
    dict(M=40, H=256, I=384, E=10, topk=2, block_m=64, wdtype="fp8", ep_size=5, ep_rank=4),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


def run_ep(p, d, ids, w, layout=moe.MOE_LAYOUT_ROWS):
    on = p.apply_router_weight_on_input
    if p.wdtype == "fp8":
        return moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, d.w13s, d.w2s,
                                 apply_router_weight_on_input=on, expert_map=d.expert_map)
    w13, w2 = d.w13, d.w2
    if layout == moe.MOE_LAYOUT_TILED:
        prob = moe.make_problem(p.M, p.H, p.I, len(p.local_experts), 1, p.block_m)  # top-k does not matter to packing
        w13, w2 = moe.moe_pack_weights(prob, 1, w13), moe.moe_pack_weights(prob, 2, w2)
    return moe.fused_experts(d.x, w13, w2, ids, w, p.block_m, apply_router_weight_on_input=on,
                             expert_map=d.expert_map, weight_layout=layout)


def oracle_ep(p, inp, ids, w):
    on, emap = p.apply_router_weight_on_input, inp.expert_map.cpu().numpy()
    if p.wdtype == "fp8":
        return oracle.fused_experts_fp8(bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                        inp.w2s.numpy(), ids, w, on_input=on, expert_map=emap)
    return oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13), bits16(inp.w2), ids, w,
                                     on_input=on, expert_map=emap)


def ep_inputs(cfg):
    p = synth.Problem(**cfg)
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    d.expert_map = inp.expert_map.to(DEV)
    return p, inp, d


@pytest.mark.parametrize("cfg", EP_CASES, ids=CASE_ID)
def test_layer_ep_matches_oracle(cfg):
    p, inp, d = ep_inputs(cfg)
    log(f"ep layer {cfg}")
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_ep(p, d, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y_ref = oracle_ep(p, inp, ids_ref, w_ref)
    assert_close(bits16(y), y_ref, TOL[p.wdtype], str(cfg))
    if p.wdtype == "bf16" and p.block_m in (16, 128, 256):
        y_t = run_ep(p, d, ids, w, moe.MOE_LAYOUT_TILED)
        torch.cuda.synchronize()
        assert torch.equal(y_t.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("block_m", [16, 128])
def test_ranks_add_up_to_the_unsharded_layer(block_m):
    base = dict(M=96, H=256, I=256, E=16, topk=4, block_m=block_m)
    p0 = synth.Problem(**base)
    inp0 = synth.make_inputs(p0, "cpu")
    d0 = to_dev(inp0)
    ids, w = moe.moe_topk(d0.logits, p0.topk)
    y_full = moe.fused_experts(d0.x, d0.w13, d0.w2, ids, w, block_m).float()
    total = torch.zeros_like(y_full)
    for rank in range(4):
        p, inp, d = ep_inputs(dict(base, ep_size=4, ep_rank=rank))
        total += run_ep(p, d, ids, w).float()
    torch.cuda.synchronize()
    # four bf16 roundings of partial sums against one: a few bf16 ulps
    err = (total - y_full).abs()
    assert bool((err <= 2e-2 * y_full.abs().clamp(min=1.0)).all()), err.max().item()


def test_full_size_ep_rank_sampled():
    name = "dsv3_ep8_rank2_prefill_m8192"
    p = synth.Problem.named(name)
    log(f"full-size {name}")
    d = synth.make_inputs(p, DEV)
    ids, w = moe.moe_topk(d.logits, p.topk)
    ys = {}
    for layout in (moe.MOE_LAYOUT_ROWS, moe.MOE_LAYOUT_TILED):
        ys[layout] = run_ep(p, d, ids, w, layout)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))
    y = ys[0]
    ids_np, w_np = oracle.topk(d.logits.cpu().numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_np)
    emap = d.expert_map.cpu().numpy()
    local = emap[ids_np] >= 0
    per_rank = np.bincount(ids_np.reshape(-1) // (p.E // p.ep_size), minlength=p.ep_size)
    assert int(np.argmax(per_rank)) == p.ep_rank and per_rank[p.ep_rank] == local.sum()
    assert np.all(y[torch.from_numpy(~local.any(1)).to(DEV)].float().cpu().numpy() == 0)
    # samples: one real row of every block of the rank's layout, tokens with the fewest and
    # the most local slots, one with exactly one, random ones up to 128
    nloc = local.sum(1)
    picks = [int(np.argmin(nloc)), int(np.argmax(nloc))] + [int(t) for t in np.nonzero(nloc == 1)[0][:1]]
    toks = sorted(set(picks + sampled.pick_tokens(ids_np, len(p.local_experts), p.block_m, expert_map=emap)))
    held = sorted(set(emap[ids_np[toks]][local[toks]].tolist()))
    sub_map = np.full(p.E, -1, np.int32)
    for i, le in enumerate(held):
        sub_map[np.nonzero(emap == le)[0][0]] = i
    sel = torch.tensor(held, device=DEV)
    log(f"full-size {name}: oracle on {len(toks)} tokens ({len(held)} local experts)")
    y_ref = oracle.fused_experts_bf16(bits16(d.x[toks]), bits16(d.w13[sel]), bits16(d.w2[sel]),
                                      ids_np[toks], w_np[toks], expert_map=sub_map)
    assert_close(bits16(y[toks]), y_ref, TOL["bf16"], name)
