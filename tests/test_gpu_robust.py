"""Workspace contents and out-of-bounds writes.

* The workspace's contents on entry do not matter: every entry point gives the
  same bits with a workspace filled with zeros and one filled with 0xFF bytes
  (NaN in every fp32 / bf16 lane, -1 in every int32).
* Nothing is written outside the caller's buffers ("vLLM modular_kernel.py
  notes", 11.4: the layer writes straight into the caller's output): y, the
  workspace, and the stage outputs (h, z, z scales, o) are allocated inside
  guard bands of a known pattern, which must be unchanged afterwards.
"""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import synth
from test_gpu_parity import DEV, log

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024  # bytes of guard band on each side


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


class Guarded:
    """A device buffer of `n` elements of `dtype` between two guard bands of 0x5A bytes."""

    def __init__(self, n: int, dtype, fill: int | None = None):
        esz = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = n * esz
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), 0x5A, dtype=torch.uint8, device=DEV)
        if fill is not None:
            self.raw[GUARD:GUARD + self.nbytes] = fill
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype)

    def view(self, *shape):
        return self.t.view(*shape)

    def intact(self) -> bool:
        return bool((self.raw[:GUARD] == 0x5A).all()) and bool((self.raw[GUARD + self.nbytes:] == 0x5A).all())


LAYERS = [
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16),
    dict(M=37, H=384, I=256, E=6, topk=3, block_m=32),
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=64),
    dict(M=300, H=512, I=384, E=5, topk=2, block_m=128),
    dict(M=300, H=512, I=384, E=3, topk=2, block_m=256),
    dict(M=300, H=512, I=384, E=3, topk=2, block_m=256, tiled=True),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8", apply_router_weight_on_input=True),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="mxfp8"),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="w4a8"),
    dict(M=130, H=640, I=384, E=16, topk=4, block_m=128, ep_size=2, ep_rank=0),
    dict(M=150, H=512, I=256, E=14, topk=3, block_m=128, wdtype="fp8", ep_size=2, ep_rank=1),
    dict(M=1000, H=256, I=256, E=8, topk=2, block_m=64, chunk_tokens=256),
    # the Mixtral shape's last round of second-GEMM tiles is split along K (576 tiles)
    dict(M=4096, H=4096, I=1792, E=8, topk=2, block_m=256, tiled=True),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


def layer_call(p: synth.Problem, d: synth.Inputs, tiled: bool):
    """(the fused_experts call taking out= and workspace=, its problem)."""
    ids, w = moe.moe_topk(d.logits.to(DEV), p.topk)
    on = p.apply_router_weight_on_input
    dev = lambda t: None if t is None else t.to(DEV)
    emap = dev(d.expert_map)
    E = len(p.local_experts)
    wdt = {"bf16": moe.MOE_W_BF16, "fp8": moe.MOE_W_FP8_E4M3_BLOCK128, "mxfp8": moe.MOE_W_MXFP8,
           "w4a8": moe.MOE_W_W4A8_MXFP4}[p.wdtype]
    layout = moe.MOE_LAYOUT_TILED if tiled else moe.MOE_LAYOUT_ROWS
    prob = moe.make_problem(p.M, p.H, p.I, E, p.topk, p.block_m, wdt, on, layout,
                            0 if emap is None else p.E, p.chunk_tokens)
    x = dev(d.x)
    if p.wdtype == "bf16":
        w13, w2, s13, s2 = dev(d.w13), dev(d.w2), None, None
        if tiled:
            rows = moe.make_problem(p.M, p.H, p.I, E, p.topk, p.block_m)
            w13, w2 = moe.moe_pack_weights(rows, 1, w13), moe.moe_pack_weights(rows, 2, w2)
    else:
        w13, w2, s13, s2 = dev(d.w13q), dev(d.w2q), dev(d.w13s), dev(d.w2s)
        if p.wdtype in ("mxfp8", "w4a8"):
            s13, s2 = moe.moe_pack_mx_scales(prob, 1, s13), moe.moe_pack_mx_scales(prob, 2, s2)

    def call(out, workspace):
        return moe.fused_experts(x, w13, w2, ids, w, p.block_m, s13, s2, apply_router_weight_on_input=on,
                                 out=out, workspace=workspace, weight_layout=layout, expert_map=emap,
                                 chunk_tokens=p.chunk_tokens)
    return call, prob


@pytest.mark.parametrize("cfg", LAYERS, ids=CASE_ID)
def test_layer_ignores_workspace_contents_and_stays_in_bounds(cfg):
    cfg = dict(cfg)
    tiled = cfg.pop("tiled", False)
    p = synth.Problem(**cfg)
    log(f"robust layer {cfg} tiled={tiled}")
    d = synth.make_inputs(p, "cpu")
    call, prob = layer_call(p, d, tiled)
    nws = max(moe.moe_workspace_bytes(prob), 256)
    results = []
    for fill in (0x00, 0xFF):
        ws = Guarded(nws, torch.uint8, fill)
        y = Guarded(p.M * p.H, torch.bfloat16, fill)
        out = call(y.view(p.M, p.H), ws.t)
        torch.cuda.synchronize()
        assert out.data_ptr() == y.t.data_ptr()
        assert ws.intact(), "write outside the workspace"
        assert y.intact(), "write outside y"
        results.append(y.t.view(torch.int16).clone())
    assert torch.equal(results[0], results[1]), "the result depends on the workspace's contents"
    assert bool(torch.isfinite(results[0].view(torch.bfloat16).float()).all())


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
def test_batched_ignores_workspace_contents_and_stays_in_bounds(wdtype):
    p = synth.Problem(M=4 * 64, H=256, I=256, E=4, topk=1, block_m=64, wdtype=wdtype)
    d = synth.make_inputs(p, "cpu")
    max_M = 64
    a = d.x.view(p.E, max_M, p.H).to(DEV)
    counts = torch.tensor([64, 0, 17, 90], dtype=torch.int32, device=DEV)
    if wdtype == "bf16":
        w13, w2, s13, s2 = d.w13.to(DEV), d.w2.to(DEV), None, None
    else:
        w13, w2, s13, s2 = d.w13q.to(DEV), d.w2q.to(DEV), d.w13s.to(DEV), d.w2s.to(DEV)
    pb = moe.make_problem(max_M, p.H, p.I, p.E, 1, p.block_m,
                          moe.MOE_W_BF16 if wdtype == "bf16" else moe.MOE_W_FP8_E4M3_BLOCK128)
    nws = max(moe.moe_batched_workspace_bytes(pb), 256)
    results = []
    for fill in (0x00, 0xFF):
        ws = Guarded(nws, torch.uint8, fill)
        out = Guarded(p.E * max_M * p.H, torch.bfloat16, fill)
        moe.moe_batched_experts(a, counts, w13, w2, p.block_m, s13, s2, out=out.view(p.E, max_M, p.H),
                                workspace=ws.t)
        torch.cuda.synchronize()
        assert ws.intact() and out.intact()
        results.append(out.t.view(torch.int16).clone())
    assert torch.equal(results[0], results[1])


@pytest.mark.parametrize("cfg", [
    dict(M=300, H=512, I=384, E=5, topk=2, block_m=128),
    dict(M=300, H=512, I=384, E=3, topk=2, block_m=256),
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16),
    dict(M=37, H=384, I=256, E=6, topk=3, block_m=64),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8"),
], ids=CASE_ID)
def test_stages_stay_in_bounds(cfg):
    # every stage entry point writes only its own output buffers, whatever they held
    p = synth.Problem(**cfg)
    log(f"robust stages {cfg}")
    d = synth.make_inputs(p, "cpu")
    fp8 = p.wdtype == "fp8"
    wdt = moe.MOE_W_FP8_E4M3_BLOCK128 if fp8 else moe.MOE_W_BF16
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, wdt)
    cap = moe.moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    ids, w = moe.moe_topk(d.logits.to(DEV), p.topk)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, p.block_m)
    x = d.x.to(DEV)
    adt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    if fp8:
        w13, w2, s13, s2 = d.w13q.to(DEV), d.w2q.to(DEV), d.w13s.to(DEV), d.w2s.to(DEV)
        xq, xs = moe.moe_quant_fp8_groups(x)
        xst = torch.empty((p.H // 128, cap), dtype=torch.float32, device=DEV)
        moe.moe_permute_scales(prob, xs, s, npp, xst)
        a1 = xq
    else:
        w13, w2, s13, s2, xst, a1 = d.w13.to(DEV), d.w2.to(DEV), None, None, None, x
    bufs = []

    def guarded(n, dtype, fill=0xFF):
        g = Guarded(n, dtype, fill)
        bufs.append(g)
        return g
    h = guarded(cap * 2 * p.I, torch.bfloat16)
    moe.moe_expert_gemm(prob, 1, a1, w13, s, e, npp, h.view(cap, 2 * p.I), xst, s13)
    z = guarded(cap * p.I, adt)
    zs = guarded((p.I // 128) * cap, torch.float32) if fp8 else None
    moe.moe_silu_and_mul(prob, h.view(cap, 2 * p.I), s, w, npp, z.view(cap, p.I),
                         None if zs is None else zs.view(p.I // 128, cap))
    if moe.moe_expert_gemm_act_supported(prob):
        z2 = guarded(cap * p.I, adt)
        zs2 = guarded((p.I // 128) * cap, torch.float32) if fp8 else None
        moe.moe_expert_gemm_act(prob, a1, xst, w13, s13, s, e, npp, w, z2.view(cap, p.I),
                                None if zs2 is None else zs2.view(p.I // 128, cap))
    o = guarded(cap * p.H, torch.bfloat16)
    gws_n = moe.lib().moe_expert_gemm_workspace_bytes(ctypes.byref(prob))
    gws = guarded(gws_n, torch.uint8) if gws_n else None
    moe.moe_expert_gemm(prob, 2, z.view(cap, p.I), w2, None, e, npp, o.view(cap, p.H),
                        None if zs is None else zs.view(p.I // 128, cap), s2,
                        workspace=None if gws is None else gws.t)
    y = guarded(p.M * p.H, torch.bfloat16)
    moe.moe_unpermute_reduce(prob, o.view(cap, p.H), inv, w, y.view(p.M, p.H))
    torch.cuda.synchronize()
    for i, g in enumerate(bufs):
        assert g.intact(), f"write outside buffer {i}"
    assert bool(torch.isfinite(y.t.float()).all())
    np.testing.assert_array_equal(y.t.view(torch.int16).cpu().numpy().shape, (p.M * p.H,))
