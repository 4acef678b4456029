"""GEMM1 that builds the routing layout itself.

For bf16 problems with block_m 16 and at most 1024 routed items (decode sizes),
fused_experts launches no align kernel: every GEMM1 workgroup rebuilds its row
block's expert and rows from the routed ids, and the workgroups of the first
column tile write the layout out for GEMM2 and the reduce. Here the layout left
in the workspace must equal moe_align_block_size's bit for bit (sorted ids with
their sentinels, expert ids, the padded total, inv_perm), and the layer must give
the bits of the stage entry points, which align first. Both weight layouts (eight-
and four-wave workgroups, so two and four passes over the ids), two hidden sizes,
routings that put many blocks on one expert, the 1024/1025-item switch and expert
maps (nothing local; a decode shard where most tokens have no local slot) are
covered.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import synth
from test_gpu_parity import DEV, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


B = 16


def routing(kind, M, k, E_route, g):
    """topk_ids [M, k] int32 (global ids when a map is used) and fp32 weights."""
    if kind == "random":
        ids = np.stack([g.choice(E_route, k, replace=False) for _ in range(M)])
    elif kind == "two":        # every token to experts 3 and 5: 32+ blocks each at M = 512
        ids = np.tile(np.array([[3, 5]]), (M, 1))
    elif kind == "one":        # every item to expert 7: one segment of many blocks
        ids = np.full((M, 1), 7)
    elif kind == "skew":       # slot 0 always expert 1, the rest random
        ids = np.stack([np.concatenate([[1], g.choice(np.arange(2, E_route), k - 1, replace=False)])
                        for _ in range(M)])
    else:
        raise ValueError(kind)
    w = g.random((M, k)).astype(np.float32)
    return (torch.from_numpy(ids.astype(np.int32)).to(DEV), torch.from_numpy(w).to(DEV))


def workspace_layout(ws, cap, R):
    """The first four regions of the layer's workspace, each on a 256-byte boundary:
    sorted ids [cap], expert ids [cap / B], the padded total [1], inv_perm [R]."""
    up = lambda b: (b + 255) // 256 * 256
    off = [0]
    for n in (cap * 4, cap // B * 4, 4, R * 4):
        off.append(off[-1] + up(n))
    part = lambda i, n: ws[off[i]:off[i] + 4 * n].view(torch.int32)
    return part(0, cap), part(1, cap // B), part(2, 1), part(3, R)


CASES = [
    # (M, k, E local, E global (0: no expert map), routing, on_input)
    (32, 8, 128, 0, "random", False),     # decode routing over 128 experts
    (128, 8, 64, 0, "random", False),     # exactly 1024 items: the largest self-aligned problem
    (205, 5, 16, 0, "random", False),     # 1025 items: the align kernel runs
    (512, 2, 8, 0, "two", False),         # two experts, 32 blocks each
    (1024, 1, 8, 0, "one", False),        # one expert, 64 blocks: ranks across every pass
    (300, 3, 12, 0, "skew", False),       # one hot expert among random ones
    (1, 1, 4, 0, "random", False),        # one item
    (40, 4, 8, 0, "random", True),        # router weight on the input
    (64, 4, 16, 32, "random", False),     # expert map: half the experts remote
    (100, 4, 4, 16, "random", False),     # expert map: nothing local (see NOTHING_LOCAL)
    (48, 8, 64, 256, "random", False),    # expert map: a decode shard, most tokens with no local slot
]
NOTHING_LOCAL = (100, 4, 4, 16)
CASE_ID = lambda c: f"M{c[0]}-k{c[1]}-E{c[2]}-G{c[3]}-{c[4]}" + ("-oninput" if c[5] else "")


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_TILED, moe.MOE_LAYOUT_ROWS], ids=["tiled", "rows"])
@pytest.mark.parametrize("case", CASES, ids=CASE_ID)
@pytest.mark.parametrize("H", [512, 384], ids=["H512", "H384"])
def test_self_aligned_layer_matches_the_aligned_stages(case, layout, H):
    M, k, E, G, kind, on_input = case
    I = 384
    log(f"self-align M={M} k={k} E={E} G={G} {kind} on_input={on_input} layout={layout} H={H}")
    g = np.random.default_rng(M * 7 + k)
    p = synth.Problem(M=M, H=H, I=I, E=E, topk=k, block_m=B)
    d = synth.make_inputs(p, DEV)
    ids, w = routing(kind, M, k, G or E, g)
    emap = None
    if G:
        held = np.full(G, -1, np.int32)
        if (M, k, E, G) != NOTHING_LOCAL:
            held[g.choice(G, E, replace=False)] = g.permutation(E)
        emap = torch.from_numpy(held).to(DEV)
    R = M * k
    w13, w2 = d.w13, d.w2
    if layout == moe.MOE_LAYOUT_TILED:
        rows = moe.make_problem(M, H, I, E, 1, B)
        w13, w2 = moe.moe_pack_weights(rows, 1, w13), moe.moe_pack_weights(rows, 2, w2)
    prob = moe.make_problem(M, H, I, E, k, B, moe.MOE_W_BF16, on_input, layout, G)
    ws = moe.workspace_for(prob, DEV)
    ws.fill_(0xAB)  # every layout entry must be written
    y = moe.fused_experts(d.x, w13, w2, ids, w, B, apply_router_weight_on_input=on_input,
                          workspace=ws, weight_layout=layout, expert_map=emap)

    # the layout the align kernel gives
    if emap is None:
        s, e, npp, inv = moe.moe_align_block_size(ids, E, B)
    else:
        s, e, npp, inv = moe.moe_align_block_size_ep(ids, emap, E, B)
    cap = s.numel()
    ws_s, ws_e, ws_n, ws_i = workspace_layout(ws, cap, R)
    torch.cuda.synchronize()
    assert int(ws_n.item()) == int(npp.item()), "padded total"
    assert torch.equal(ws_e, e), "expert ids"
    assert torch.equal(ws_s, s), "sorted ids"
    assert torch.equal(ws_i, inv.view(-1)), "inv_perm"

    # the stages, launched one by one on the aligned layout
    z = torch.empty((cap, I), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    sp = moe.make_problem(M, H, I, E, k, B, moe.MOE_W_BF16, on_input, layout)
    moe.moe_expert_gemm_act(sp, d.x, None, w13, None, s, e, npp, w, z)
    moe.moe_expert_gemm(sp, 2, z, w2, None, e, npp, o)
    y_st = torch.empty_like(d.x)
    moe.moe_unpermute_reduce(sp, o, inv, w, y_st)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_st.view(torch.int16))
    if G and not bool((emap >= 0).any()):
        assert not bool(y.view(torch.int16).any()), "no local expert: y is zero"


def test_self_aligned_layer_twice_with_fewer_items():
    # the second call reuses the workspace of the first with fewer items; nothing of
    # the first layout may leak into the second
    H, I, E = 256, 256, 32
    g = np.random.default_rng(11)
    p = synth.Problem(M=120, H=H, I=I, E=E, topk=8, block_m=B)
    d = synth.make_inputs(p, DEV)
    ws = moe.workspace_for(moe.make_problem(120, H, I, E, 8, B), DEV)
    for M in (120, 9):
        ids, w = routing("random", M, 8, E, g)
        x = d.x[:M].contiguous()
        y = moe.fused_experts(x, d.w13, d.w2, ids, w, B, workspace=ws)
        y_new = moe.fused_experts(x, d.w13, d.w2, ids, w, B)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_new.view(torch.int16)), f"M={M}"
