"""Batched-experts form ([E, max_M, H] batches with per-expert counts): matches
the oracle element by element on every GEMM path, never reads rows past a count
(they hold NaN here), writes 0 there, and gives the same bits on tiled weights."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
import synth
from hostutil import bits16, bits8
from test_gpu_parity import DEV, TOL, assert_close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


CASES = [
    dict(E=8, max_M=32, H=256, I=512, block_m=16, counts="random"),
    dict(E=128, max_M=32, H=2048, I=768, block_m=16, counts="decode"),     # decode-shaped batches
    dict(E=5, max_M=300, H=640, I=384, block_m=128, counts="random"),
    dict(E=3, max_M=256, H=512, I=384, block_m=256, counts="edges"),
    dict(E=6, max_M=70, H=384, I=256, block_m=32, counts="random"),
    dict(E=6, max_M=150, H=512, I=256, block_m=128, counts="random", wdtype="fp8"),
    dict(E=4, max_M=40, H=256, I=384, block_m=64, counts="edges", wdtype="fp8"),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


def make_case(c):
    wdtype = c.get("wdtype", "bf16")
    E, max_M = c["E"], c["max_M"]
    p = synth.Problem(M=max_M, H=c["H"], I=c["I"], E=E, topk=1, wdtype=wdtype, block_m=c["block_m"])
    inp = synth.make_inputs(p, "cpu")
    g = np.random.default_rng(E * max_M)
    if c["counts"] == "edges":   # empty, full, over-full, negative, partial
        counts = np.array([0, max_M, max_M + 5, -2, 1, max_M - 1][:E], np.int32)
    elif c["counts"] == "decode":
        counts = np.minimum(g.poisson(2.0, E), max_M).astype(np.int32)
    else:
        counts = g.integers(0, max_M + 1, E).astype(np.int32)
        counts[0] = 0
    a = torch.randn((E, max_M, p.H), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    n = np.clip(counts, 0, max_M)
    for e in range(E):   # rows past the count hold NaN: they must not be read
        a[e, n[e]:] = float("nan")
    return p, inp, a, counts, n


def run(p, inp, a, counts, layout=moe.MOE_LAYOUT_ROWS):
    cnt = torch.from_numpy(counts).to(DEV)
    if p.wdtype == "fp8":
        return moe.moe_batched_experts(a.to(DEV), cnt, inp.w13q.to(DEV), inp.w2q.to(DEV), p.block_m,
                                       inp.w13s.to(DEV), inp.w2s.to(DEV))
    w13, w2 = inp.w13.to(DEV), inp.w2.to(DEV)
    if layout == moe.MOE_LAYOUT_TILED:
        prob = moe.make_problem(1, p.H, p.I, p.E, 1, p.block_m)
        w13, w2 = moe.moe_pack_weights(prob, 1, w13), moe.moe_pack_weights(prob, 2, w2)
    return moe.moe_batched_experts(a.to(DEV), cnt, w13, w2, p.block_m, weight_layout=layout)


@pytest.mark.parametrize("c", CASES, ids=CASE_ID)
def test_batched_matches_oracle(c):
    p, inp, a, counts, n = make_case(c)
    log(f"batched {c}")
    out = run(p, inp, a, counts)
    torch.cuda.synchronize()
    a_clean = bits16(a).copy()
    for e in range(p.E):
        a_clean[e, n[e]:] = 0
    if p.wdtype == "fp8":
        ref = oracle.batched_experts_fp8(a_clean, n, bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                         inp.w2s.numpy())
    else:
        ref = oracle.batched_experts_bf16(a_clean, n, bits16(inp.w13), bits16(inp.w2))
    got = bits16(out)
    for e in range(p.E):
        assert np.all(got[e, n[e]:] == 0), f"expert {e}: rows past the count not zero"
        if n[e]:
            assert_close(got[e, :n[e]], ref[e, :n[e]], TOL[p.wdtype], f"{c} expert {e}")
    if p.wdtype == "bf16" and p.block_m in (16, 128, 256):
        out_t = run(p, inp, a, counts, moe.MOE_LAYOUT_TILED)
        torch.cuda.synchronize()
        assert torch.equal(out_t.view(torch.int16), out.view(torch.int16))
