"""Parity of the HIP path (through the C ABI) with the CPU oracle.

* Router ids, the aligned layout and the fp8 activation codes are compared
  bit for bit; router weights within 1e-6 (fp32 exp and division of k <= 32
  terms: a few ulp of a value <= 1).
* y is compared element by element: |y - y_ref| <= tol * max(1, |y_ref|) with
  tol = 2e-2 for bf16 and 6e-2 for fp8.
* Full-size workloads are checked on sampled tokens, which the oracle computes
  one by one from host copies of the inputs those tokens touch.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import sampled
import synth
from hostutil import bf16_f64, bits16, bits8

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"bf16": 2e-2, "fp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def log(msg):
    print(msg, flush=True)


def to_dev(inp: synth.Inputs) -> synth.Inputs:
    return synth.Inputs(*[None if t is None else t.to(DEV) for t in (
        inp.x, inp.logits, inp.w13, inp.w2, inp.w13q, inp.w13s, inp.w2q, inp.w2s)])


def route_gpu(p: synth.Problem, logits, score_bias):
    """The workload's router on the GPU: softmax top-k or the grouped / sigmoid router."""
    if p.scoring == "softmax" and p.n_group == 1 and score_bias is None and p.routed_scale == 1.0:
        return moe.moe_topk(logits, p.topk)
    return moe.moe_topk_grouped(logits, p.topk, p.scoring, True, p.n_group, p.topk_group, score_bias,
                                p.routed_scale)


def route_oracle(p: synth.Problem, logits: np.ndarray, score_bias):
    if p.scoring == "softmax" and p.n_group == 1 and score_bias is None and p.routed_scale == 1.0:
        return oracle.topk(logits, p.topk)
    return oracle.topk_grouped(logits, p.topk, p.scoring, True, p.n_group, p.topk_group,
                               None if score_bias is None else score_bias.cpu().numpy(), p.routed_scale)


def router_inputs(p: synth.Problem):
    """The workload's logits and correction bias, drawn with small H and I (the same draws)."""
    small = synth.Problem(M=p.M, H=128, I=128, E=p.E, topk=p.topk, bias_std=p.bias_std, seed=p.seed,
                          score_bias_std=p.score_bias_std)
    inp = synth.make_inputs(small, "cpu")
    return inp.logits, inp.score_bias


def run_layer(p: synth.Problem, d: synth.Inputs, ids, w, out=None):
    if p.wdtype == "fp8":
        return moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, d.w13s, d.w2s,
                                 apply_router_weight_on_input=p.apply_router_weight_on_input,
                                 out=out, chunk_tokens=p.chunk_tokens)
    return moe.fused_experts(d.x, d.w13, d.w2, ids, w, p.block_m,
                             apply_router_weight_on_input=p.apply_router_weight_on_input, out=out,
                             chunk_tokens=p.chunk_tokens)


def oracle_layer(p, inp_cpu, ids, w, t0=0, t1=None):
    on = p.apply_router_weight_on_input
    if p.wdtype == "fp8":
        return oracle.fused_experts_fp8(bits16(inp_cpu.x), bits8(inp_cpu.w13q),
                                        inp_cpu.w13s.numpy(), bits8(inp_cpu.w2q),
                                        inp_cpu.w2s.numpy(), ids, w, on_input=on, t0=t0, t1=t1)
    return oracle.fused_experts_bf16(bits16(inp_cpu.x), bits16(inp_cpu.w13), bits16(inp_cpu.w2),
                                     ids, w, on_input=on, t0=t0, t1=t1)


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float, what: str):
    a, b = bf16_f64(y_gpu), bf16_f64(y_ref)
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    err = np.abs(a - b)
    lim = tol * np.maximum(1.0, np.abs(b))
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:4].tolist()}, "
                           f"max err {err.max():.4g}")


# ------------------------------------------------------------------ router ---

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_router_bit_exact(name):
    p = synth.Problem.named(name)
    log(f"router {name}")
    logits, sb = router_inputs(p)
    ids, w = route_gpu(p, logits.to(DEV), None if sb is None else sb.to(DEV))
    ids_ref, w_ref = route_oracle(p, logits.numpy(), sb)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6 * max(1.0, p.routed_scale)


def test_router_ties_and_unnormalised():
    logits = torch.zeros((8, 16), dtype=torch.float32)
    logits[:, 3] = 1.0
    logits[:, 7] = 1.0
    logits[4:, :] = torch.randn(4, 16, generator=torch.Generator().manual_seed(3))
    for renorm in (True, False):
        ids, w = moe.moe_topk(logits.to(DEV), 4, renormalize=renorm)
        ids_ref, w_ref = oracle.topk(logits.numpy(), 4, renormalize=renorm)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6


def test_router_nan_logits():
    # a NaN logit ranks below every number (the oracle's reading); a token whose logits
    # are all NaN gets ids 0..k-1 and NaN weights, so its y row is NaN, not silently 0
    g = torch.Generator().manual_seed(11)
    logits = torch.randn(64, 256, generator=g)
    logits[0, :200] = float("nan")
    logits[1, [3, 77, 130, 255]] = float("nan")
    logits[2, :] = float("nan")
    logits[3, 5] = float("-inf")
    logits[3, 6] = float("nan")
    for renorm in (True, False):
        ids, w = moe.moe_topk(logits.to(DEV), 8, renormalize=renorm)
        ids_ref, w_ref = oracle.topk(logits.numpy(), 8, renormalize=renorm)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        wg = w.cpu().numpy()
        assert np.array_equal(np.isnan(wg), np.isnan(w_ref))
        ok = ~np.isnan(w_ref)
        assert np.abs(wg[ok] - w_ref[ok]).max() <= 1e-6
    ids, w = moe.moe_topk_grouped(logits.to(DEV), 8, "sigmoid", True, 8, 4,
                                  torch.zeros(256, device=DEV), 2.5)
    ids_ref, _ = oracle.topk_grouped(logits.numpy(), 8, "sigmoid", True, 8, 4, np.zeros(256, np.float32), 2.5)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert ((ids >= 0) & (ids < 256)).all()
    # through the layer: finite rows stay finite, the all-NaN token's row is NaN
    p = synth.Problem(M=64, H=256, I=256, E=256, topk=8, block_m=16)
    d = to_dev(synth.make_inputs(synth.Problem(M=64, H=256, I=256, E=256, topk=8), "cpu"))
    ids, w = moe.moe_topk(logits.to(DEV), 8)
    y = run_layer(p, d, ids, w).float()
    torch.cuda.synchronize()
    assert bool(torch.isnan(y[2]).all())
    keep = torch.ones(64, dtype=torch.bool)
    keep[2] = False
    assert bool(torch.isfinite(y[keep.to(DEV)]).all())


def test_binding_rejects_mis_shaped_weight_scales():
    p = synth.Problem(M=40, H=256, I=256, E=4, topk=2, block_m=64, wdtype="fp8")
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    for s13, s2 in ((d.w13s[:1], d.w2s), (d.w13s, d.w2s.transpose(1, 2).contiguous()[:, :1]),
                    (d.w13s, d.w2s[:2])):
        with pytest.raises(ValueError, match="scale"):
            moe.fused_experts(d.x, d.w13q, d.w2q, ids, w, p.block_m, s13.contiguous(), s2.contiguous())


# ------------------------------------------------------------------- align ---

def check_align(ids_np: np.ndarray, E: int, B: int):
    ids = torch.from_numpy(ids_np).to(DEV)
    s, x, npp, inv = moe.moe_align_block_size(ids, E, B)
    rs, rx, rnpp, rinv = oracle.align(ids_np, E, B)
    assert int(npp.item()) == rnpp
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(x.cpu().numpy(), rx)
    assert np.array_equal(inv.cpu().numpy(), rinv)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_align_bit_exact_workloads(name):
    p = synth.Problem.named(name)
    log(f"align {name}")
    logits, sb = router_inputs(p)
    ids, _ = route_oracle(p, logits.numpy(), sb)
    for B in sorted({p.block_m, 16, 64, 128, 256}):
        check_align(ids, p.E, B)


def test_align_edge_cases():
    g = np.random.default_rng(0)
    check_align(np.zeros((300, 1), np.int32), 4, 16)                     # all to one expert
    check_align(np.tile(np.arange(8, dtype=np.int32), (5, 1)), 8, 32)     # E == topk
    check_align(np.array([[3, 1]], np.int32), 8, 128)                     # M = 1
    ids = np.stack([g.choice(256, 8, replace=False) for _ in range(3000)]).astype(np.int32)
    check_align(ids, 256, 64)
    skew = np.minimum(g.geometric(0.05, (5000, 4)), 255).astype(np.int32)  # heavy skew, dupes ok
    check_align(skew, 256, 16)



def test_align_many_workgroups_boundaries():
    # from 8192 items on, chunks of 1024 items are counted and placed by separate
    # workgroups: both sides of that switch, ragged last chunks, chunk boundaries
    # inside one expert's run (ids in ascending order) and a single expert
    g = np.random.default_rng(3)
    for M, k, E, B in ((8191, 1, 256, 16), (8192, 1, 256, 16), (8193, 1, 7, 128), (2049, 4, 5, 256),
                       (9000, 8, 256, 64), (9000, 1, 1, 128)):
        log(f"align many-wg M={M} k={k} E={E} B={B}")
        ids = np.stack([g.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
        check_align(ids, E, B)
        check_align(np.sort(ids, axis=0), E, B)



@pytest.mark.parametrize("block_m,wdtype", [(128, "bf16"), (256, "bf16"), (128, "fp8")])
def test_gemm_real_rows_around_padding_groups(block_m, wdtype):
    # hand-made layouts in which padding rows (sorted id >= M*topk) fill whole 32-row
    # groups before, between and after real rows, and whole blocks: every real row
    # still gets its product in both GEMMs (groups of padding alone are not multiplied)
    M, topk, E, H, I = 96, 2, 3, 512, 256
    R, B = M * topk, block_m
    fp8 = wdtype == "fp8"
    p = synth.Problem(M=M, H=H, I=I, E=E, topk=topk, block_m=B, wdtype=wdtype)
    log(f"padding groups block_m={B} {wdtype}")
    d = to_dev(synth.make_inputs(p, "cpu"))
    prob = moe.make_problem(M, H, I, E, topk, B, moe.MOE_W_FP8_E4M3_BLOCK128 if fp8 else moe.MOE_W_BF16)
    cap = moe.moe_align_capacity(M, topk, E, B)
    nb = cap // B
    assert nb >= 4
    rows = {0: (0, list(range(32, 64)) + [B - 1]),   # block: (expert, real rows)
            1: (1, [0]),
            2: (2, []),
            3: (0, [0, 64, 101] + ([130, 200, 255] if B == 256 else []))}
    for b in range(4, nb):
        rows[b] = (1, list(range(B - 32, B))) if b % 2 == 0 else (-1, [])
    g = np.random.default_rng(11)
    items = iter(g.permutation(R))
    sorted_ids = np.full(cap, R, np.int32)
    expert_ids = np.empty(nb, np.int32)
    for b, (e, rr) in rows.items():
        expert_ids[b] = e
        for r in rr:
            sorted_ids[b * B + r] = next(items)
    s = torch.from_numpy(sorted_ids).to(DEV)
    ex = torch.from_numpy(expert_ids).to(DEV)
    npp = torch.tensor([cap], dtype=torch.int32, device=DEV)
    h = torch.empty((cap, 2 * I), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    zg = torch.Generator().manual_seed(2)
    z = torch.randn(cap, I, generator=zg).to(torch.bfloat16)
    if fp8:
        xq, xs = moe.moe_quant_fp8_groups(d.x)
        xst = torch.empty((H // 128, cap), dtype=torch.float32, device=DEV)
        moe.moe_permute_scales(prob, xs, s, npp, xst)
        moe.moe_expert_gemm(prob, 1, xq, d.w13q, s, ex, npp, h, xst, d.w13s)
        zq, zs = moe.moe_quant_fp8_groups(z.to(DEV))
        zst = zs.t().contiguous()  # [I/128, cap], by position
        moe.moe_expert_gemm(prob, 2, zq, d.w2q, s, ex, npp, o, zst, d.w2s)
        xqb, xsb, zqb, zsb = bits8(xq), xs.cpu().numpy(), bits8(zq), zs.cpu().numpy()
        w13qb, w13sb, w2qb, w2sb = bits8(d.w13q), d.w13s.cpu().numpy(), bits8(d.w2q), d.w2s.cpu().numpy()
        ref1 = lambda r, e: oracle.gemm_fp8(xqb[r // topk], xsb[r // topk], w13qb[e], w13sb[e])
        ref2 = lambda pos, e: oracle.gemm_fp8(zqb[pos], zsb[pos], w2qb[e], w2sb[e])
        tol = 6e-2
    else:
        moe.moe_expert_gemm(prob, 1, d.x, d.w13, s, ex, npp, h)
        moe.moe_expert_gemm(prob, 2, z.to(DEV), d.w2, s, ex, npp, o)
        xb, w13b, w2b, zb = bits16(d.x), bits16(d.w13), bits16(d.w2), bits16(z)
        ref1 = lambda r, e: oracle.gemm1_bf16(xb[r // topk], w13b[e])
        ref2 = lambda pos, e: oracle.gemm2_bf16(zb[pos], w2b[e])
        tol = 2e-2
    torch.cuda.synchronize()
    hb, ob = bits16(h), bits16(o)
    checked = 0
    for pos in range(cap):
        r, e = int(sorted_ids[pos]), int(expert_ids[pos // B])
        if r >= R or e < 0:
            continue
        for got, ref in ((hb[pos], ref1(r, e)), (ob[pos], ref2(pos, e))):
            g64, r64 = bf16_f64(got), bf16_f64(ref)
            assert np.all(np.abs(g64 - r64) <= tol * np.maximum(1.0, np.abs(r64))), (pos, r, e)
        checked += 1
    assert checked == sum(len(rr) for e, rr in rows.values() if e >= 0)

# ------------------------------------------------------------------- quant ---

def test_quant_fp8_bit_exact():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(515, 7168, generator=g) * torch.exp2(torch.randint(-8, 8, (515, 1), generator=g))
    x[3, 128:256] = 0.0
    x[4, :5] = -0.0
    xb = x.to(torch.bfloat16)
    q, s = moe.moe_quant_fp8_groups(xb.to(DEV))
    q_ref, s_ref = oracle.quant_groups_fp8(xb.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(bits8(q), q_ref)


def test_permute_scales_bit_exact():
    # per-token group scales follow their rows into the expert-sorted order,
    # stored group-major; padding positions get 0, later positions untouched
    M, k, E, B, H = 300, 4, 16, 128, 640
    g = torch.Generator().manual_seed(5)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(M)]).to(torch.int32)
    scale = torch.rand(M, H // 128, generator=g) + 0.5
    prob = moe.make_problem(M, H, 256, E, k, B, moe.MOE_W_FP8_E4M3_BLOCK128)
    s, e, npp, inv = moe.moe_align_block_size(ids.to(DEV), E, B)
    cap = s.numel()
    out = torch.full((H // 128, cap), float("nan"), device=DEV)
    moe.moe_permute_scales(prob, scale.to(DEV), s, npp, out)
    sn, n = s.cpu().numpy(), int(npp.item())
    ref = np.zeros((H // 128, n), np.float32)
    real = sn[:n] < M * k
    ref[:, real] = scale.numpy()[sn[:n][real] // k].T
    o = out.cpu().numpy()
    assert n < cap and np.array_equal(o[:, :n], ref)
    assert np.all(np.isnan(o[:, n:]))


@pytest.mark.parametrize("cfg", [
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=64, H=384, I=256, E=3, topk=2, block_m=32, wdtype="fp8"),
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8", apply_router_weight_on_input=True),
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=128),
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=16),
    dict(M=300, H=512, I=384, E=3, topk=2, block_m=256),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_stages_compose_to_fused(cfg):
    # the exported stage entry points, launched one by one, give fused_experts' bits
    p = synth.Problem(**cfg)
    log(f"stages {cfg}")
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    y_fused = run_layer(p, d, ids, w)
    fp8 = p.wdtype == "fp8"
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m,
                            moe.MOE_W_FP8_E4M3_BLOCK128 if fp8 else moe.MOE_W_BF16, p.apply_router_weight_on_input)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, p.block_m)
    cap = s.numel()
    a1, a1s = d.x, None
    if fp8:
        a1, xs = moe.moe_quant_fp8_groups(d.x)
        a1s = torch.empty((p.H // 128, cap), dtype=torch.float32, device=DEV)
        moe.moe_permute_scales(prob, xs, s, npp, a1s)
    z = torch.empty((cap, p.I), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16, device=DEV)
    zs = torch.empty((p.I // 128, cap), dtype=torch.float32, device=DEV) if fp8 else None
    if moe.moe_expert_gemm_act_supported(prob):
        moe.moe_expert_gemm_act(prob, a1, a1s, d.w13q if fp8 else d.w13, d.w13s, s, e, npp, w, z, zs)
    else:
        h = torch.empty((cap, 2 * p.I), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_gemm(prob, 1, a1, d.w13q if fp8 else d.w13, s, e, npp, h, a1s, d.w13s)
        moe.moe_silu_and_mul(prob, h, s, w, npp, z, zs)
    o = torch.empty((cap, p.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_expert_gemm(prob, 2, z, d.w2q if fp8 else d.w2, None, e, npp, o, zs, d.w2s,
                        workspace=moe.gemm_workspace_for(prob, DEV))
    y = torch.empty_like(d.x)
    moe.moe_unpermute_reduce(prob, o, inv, w, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_fused)


@pytest.mark.parametrize("cfg", [
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=200, H=384, I=640, E=6, topk=2, block_m=128, wdtype="fp8"),       # 5 column blocks
    dict(M=300, H=256, I=128, E=4, topk=2, block_m=128, wdtype="fp8",        # 2 K stages
         apply_router_weight_on_input=True),
    dict(M=1, H=512, I=256, E=4, topk=2, block_m=128, wdtype="fp8"),         # one token
    dict(M=150, H=512, I=384, E=7, topk=3, block_m=128, wdtype="bf16"),       # 2 column tiles, ragged
    dict(M=300, H=256, I=640, E=5, topk=2, block_m=256, wdtype="bf16"),       # 5 column tiles
    dict(M=90, H=384, I=256, E=4, topk=2, block_m=256, wdtype="bf16",
         apply_router_weight_on_input=True),
    dict(M=1, H=256, I=128, E=4, topk=2, block_m=128, wdtype="bf16"),         # one token, tail tile
    dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16, wdtype="bf16"),      # decode shape
    dict(M=21, H=384, I=256, E=6, topk=3, block_m=16, wdtype="bf16",          # 128-byte chunks
         apply_router_weight_on_input=True),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_gemm_act_matches_gemm_then_act(cfg):
    # the fused SiLU epilogue gives the bits of GEMM1 (h in bf16) followed by
    # the separate activation (+ quantisation for fp8) pass
    p = synth.Problem(**cfg)
    log(f"gemm_act {cfg}")
    fp8 = p.wdtype == "fp8"
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m,
                            moe.MOE_W_FP8_E4M3_BLOCK128 if fp8 else moe.MOE_W_BF16,
                            p.apply_router_weight_on_input)
    assert moe.moe_expert_gemm_act_supported(prob)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, p.block_m)
    cap, n = s.numel(), int(npp.item())
    h = torch.empty((cap, 2 * p.I), dtype=torch.bfloat16, device=DEV)
    if fp8:
        xq, xs = moe.moe_quant_fp8_groups(d.x)
        xst = torch.empty((p.H // 128, cap), dtype=torch.float32, device=DEV)
        moe.moe_permute_scales(prob, xs, s, npp, xst)
        x, w13, w13s = xq, d.w13q, d.w13s
        zdt = torch.float8_e4m3fn
        zs0 = torch.zeros((p.I // 128, cap), dtype=torch.float32, device=DEV)
        zs1 = torch.zeros_like(zs0)
    else:
        x, xst, w13, w13s = d.x, None, d.w13, None
        zdt = torch.bfloat16
        zs0 = zs1 = None
    moe.moe_expert_gemm(prob, 1, x, w13, s, e, npp, h, xst, w13s)
    z0 = torch.zeros((cap, p.I), dtype=zdt, device=DEV)
    moe.moe_silu_and_mul(prob, h, s, w, npp, z0, zs0)
    z1 = torch.full_like(z0, 1.0) if not fp8 else torch.zeros_like(z0)
    moe.moe_expert_gemm_act(prob, x, xst, w13, w13s, s, e, npp, w, z1, zs1)
    torch.cuda.synchronize()
    assert torch.equal(z0[:n].view(torch.uint8), z1[:n].view(torch.uint8))
    if fp8:
        assert torch.equal(zs0[:, :n], zs1[:, :n])


def test_gemm_act_unsupported_cases():
    for kw in (dict(wdtype=moe.MOE_W_BF16, block_m=64, H=512), dict(wdtype=moe.MOE_W_BF16, block_m=32, H=512),
               dict(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=64, H=512),
               dict(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=128, H=128)):
        prob = moe.make_problem(64, kw["H"], 256, 8, 2, kw["block_m"], kw["wdtype"])
        assert not moe.moe_expert_gemm_act_supported(prob)


def test_stage_binding_rejects_row_major_scales():
    # the GEMM reads a_scale as [K/128, cap]; a per-token [M, K/128] buffer is
    # refused by the binding before anything is launched
    p = synth.Problem(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8")
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, moe.MOE_W_FP8_E4M3_BLOCK128)
    s, e, npp, inv = moe.moe_align_block_size(ids, p.E, p.block_m)
    xq, xs = moe.moe_quant_fp8_groups(d.x)
    h = torch.empty((s.numel(), 2 * p.I), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="a_scale"):
        moe.moe_expert_gemm(prob, 1, xq, d.w13q, s, e, npp, h, xs, d.w13s)


# ------------------------------------------------------------- full layer ---

SMALL = [
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16),                 # tiny workload
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=32),
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=64),
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=128),
    dict(M=37, H=384, I=256, E=6, topk=3, block_m=32),                 # ragged tails
    dict(M=37, H=384, I=256, E=6, topk=3, block_m=64),
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=128),
    dict(M=130, H=640, I=384, E=5, topk=2, block_m=16),
    dict(M=1, H=256, I=256, E=4, topk=2, block_m=16),                  # a single token
    dict(M=1, H=256, I=256, E=4, topk=2, block_m=128),
    dict(M=24, H=256, I=256, E=4, topk=4, block_m=32),                 # E == topk
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=64, apply_router_weight_on_input=True),
    dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16),              # decode workload
    dict(M=300, H=512, I=384, E=3, topk=2, block_m=256),               # 256-row blocks
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=256),
]
FP8_SMALL = [
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=32, wdtype="fp8"),
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8"),
    dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"),
    dict(M=40, H=256, I=384, E=5, topk=2, block_m=64, wdtype="fp8",
         apply_router_weight_on_input=True),
    # tail tile of 128 valid weight rows in GEMM2 (N = H = 3 x 128), 3 K stages in GEMM1
    dict(M=200, H=384, I=640, E=6, topk=2, block_m=128, wdtype="fp8"),
    # a single K stage in GEMM2 (K = I = 128)
    dict(M=90, H=256, I=128, E=4, topk=2, block_m=128, wdtype="fp8"),
    dict(M=64, H=384, I=256, E=3, topk=2, block_m=32, wdtype="fp8"),
]


@pytest.mark.parametrize("cfg", SMALL + FP8_SMALL, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_small_elementwise(cfg):
    p = synth.Problem(**cfg)
    log(f"layer {cfg}")
    inp = synth.make_inputs(p, "cpu")
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    d = to_dev(inp)
    ids, w = moe.moe_topk(d.logits, p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y = run_layer(p, d, ids, w)
    torch.cuda.synchronize()
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6
    y_ref = oracle_layer(p, inp, ids_ref, w_ref)
    assert_close(bits16(y), y_ref, TOL[p.wdtype], str(cfg))


def test_layer_all_tokens_one_expert_and_in_place():
    p = synth.Problem(M=200, H=256, I=256, E=8, topk=2, block_m=64)
    inp = synth.make_inputs(p, "cpu")
    ids_np = np.tile(np.array([[5, 2]], np.int32), (p.M, 1))
    w_np = np.tile(np.array([[0.75, 0.25]], np.float32), (p.M, 1))
    d = to_dev(inp)
    x_copy = d.x.clone()
    y = run_layer(p, d, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), out=d.x)
    torch.cuda.synchronize()
    assert y.data_ptr() == d.x.data_ptr()
    assert not torch.equal(x_copy, d.x)
    y_ref = oracle_layer(p, inp, ids_np, w_np)
    assert_close(bits16(y), y_ref, TOL["bf16"], "one expert, in place")


def test_layer_deterministic():
    p = synth.Problem(M=300, H=512, I=384, E=16, topk=4, block_m=64)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    a = run_layer(p, d, ids, w)
    b = run_layer(p, d, ids, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_token_permutation_equivariance():
    # permuting tokens permutes y rows; routing and tiles change, so compare
    # to tolerance rather than bits
    p = synth.Problem(M=96, H=256, I=256, E=6, topk=2, block_m=32)
    d = to_dev(synth.make_inputs(p, "cpu"))
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_layer(p, d, ids, w)
    perm = torch.randperm(p.M, generator=torch.Generator().manual_seed(1)).to(DEV)
    dp = synth.Inputs(d.x[perm].contiguous(), d.logits[perm].contiguous(), d.w13, d.w2)
    yp = run_layer(p, dp, ids[perm].contiguous(), w[perm].contiguous())
    torch.cuda.synchronize()
    assert_close(bits16(yp), bits16(y[perm]), 1e-2, "permuted tokens")


# --------------------------------------------------- full-size, sampled ---

def sampled_check(name, **overrides):
    p = synth.Problem.named(name, **overrides)
    log(f"full-size {name} {overrides}: generating inputs on the device")
    d = synth.make_inputs(p, DEV)
    ids, w = route_gpu(p, d.logits, d.score_bias)
    y = run_layer(p, d, ids, w)
    torch.cuda.synchronize()
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref = route_oracle(p, d.logits.cpu().numpy(), d.score_bias)
    assert np.array_equal(ids_np, ids_ref)
    assert np.abs(w_np - w_ref).max() <= 1e-6 * max(1.0, p.routed_scale)
    # one real row of every block of the layout (every tile), single-token experts,
    # first and last tokens, random ones up to 128
    toks = sampled.pick_tokens(ids_ref, p.E, p.block_m, chunk=p.chunk_tokens)
    experts, sub_ids = sampled.expert_subset(ids_ref, toks, p.E)
    sel = torch.tensor(experts, device=DEV)
    log(f"full-size {name}: oracle on {len(toks)} tokens ({len(experts)} experts)")
    sub = synth.Inputs(d.x[toks].cpu(), None,
                       None if d.w13 is None else d.w13[sel].cpu(),
                       None if d.w2 is None else d.w2[sel].cpu(),
                       None if d.w13q is None else d.w13q[sel].cpu(),
                       None if d.w13s is None else d.w13s[sel].cpu(),
                       None if d.w2q is None else d.w2q[sel].cpu(),
                       None if d.w2s is None else d.w2s[sel].cpu())
    y_ref = oracle_layer(p, sub, sub_ids, w_ref[toks])
    assert_close(bits16(y[toks]), y_ref, TOL[p.wdtype], name)
    assert bool(torch.isfinite(y.float()).all())


@pytest.mark.parametrize("name", ["mixtral_prefill_m4096", "dsv3_skewed_prefill_m8192",
                                  "fp8_block_m4096", "dsv3_grouped_prefill_m8192",
                                  "mixtral_prefill_m32768_chunk16k"])
def test_layer_full_size_sampled(name):
    sampled_check(name)


def test_layer_full_size_sampled_mixtral_256_row_blocks():
    # the Mixtral shape in 256-row blocks (256 x 256 tiles, split-K tail of GEMM2)
    sampled_check("mixtral_prefill_m4096", block_m=256)


# ------------------------------------------------------------- chunking ---

CHUNKED = [
    dict(M=1000, H=256, I=256, E=8, topk=2, block_m=64, chunk_tokens=256),          # ragged last chunk
    dict(M=700, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8", chunk_tokens=300),
    dict(M=333, H=384, I=256, E=6, topk=2, block_m=16, chunk_tokens=100,
         apply_router_weight_on_input=True),
    dict(M=600, H=512, I=384, E=3, topk=2, block_m=256, chunk_tokens=512),
    dict(M=64, H=256, I=512, E=8, topk=2, block_m=16, chunk_tokens=64),             # one chunk
]


@pytest.mark.parametrize("cfg", CHUNKED, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_chunked(cfg):
    # chunks run the layer on token ranges one after another: each token's result is
    # the oracle's (within tolerance) and close to the one-pass result; in place too
    p = synth.Problem(**cfg)
    log(f"chunked {cfg}")
    inp = synth.make_inputs(p, "cpu")
    d = to_dev(inp)
    ids, w = moe.moe_topk(d.logits, p.topk)
    y = run_layer(p, d, ids, w)
    one = run_layer(synth.Problem(**dict(cfg, chunk_tokens=0)), d, ids, w)
    x_copy = d.x.clone()
    y_in = run_layer(p, d, ids, w, out=d.x)
    torch.cuda.synchronize()
    assert torch.equal(y_in, y) and not torch.equal(d.x, x_copy)
    ids_ref, w_ref = oracle.topk(inp.logits.numpy(), p.topk)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    y_ref = oracle_layer(p, inp, ids_ref, w_ref)
    assert_close(bits16(y), y_ref, TOL[p.wdtype], str(cfg))
    assert_close(bits16(y), bits16(one), TOL[p.wdtype], "chunked vs one pass")
    if p.chunk_tokens >= p.M:
        assert torch.equal(y, one)
