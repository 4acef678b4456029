"""The layer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Nothing the library enqueues is a memset (the split-K counters and every other
buffer that must start at zero are cleared by kernels), and the host never reads
device values, so `moe_topk` + `fused_experts` (with a preallocated workspace)
and `moe_topk` + `fused_experts_static` (no workspace at all) can be captured.
Each case replays the graph several times, with the output cleared and other
eager work run between the replays, and every replay must give the bits of the
eager call on the same inputs.
"""
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


CASES = [
    # decode shape on tiled weights: the weight-streaming kernels
    (dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16), "tiled", False),
    # 128-row DMA tiles with the split-K tail of the second GEMM (counters zeroed by a kernel)
    (dict(M=300, H=512, I=384, E=5, topk=2, block_m=128), "tiled", False),
    (dict(M=300, H=512, I=384, E=3, topk=2, block_m=256), "rows", False),
    # fp8: the activation quantiser, the scale permute and the persistent kernel
    (dict(M=150, H=512, I=256, E=7, topk=3, block_m=128, wdtype="fp8"), "rows", False),
    # token chunks: the pipeline once per chunk inside one graph
    (dict(M=1000, H=256, I=256, E=8, topk=2, block_m=64, chunk_tokens=256), "rows", False),
    # the no-allocation entry point
    (dict(M=300, H=512, I=384, E=5, topk=2, block_m=128), "tiled", True),
    (dict(M=32, H=2048, I=768, E=128, topk=8, block_m=16), "tiled", True),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c[0].items()) + f"-{c[1]}" + ("-static" if c[2] else "")


@pytest.mark.parametrize("case", CASES, ids=CASE_ID)
def test_captured_layer_replays_bit_exactly(case):
    cfg, layout, static = case
    p = synth.Problem(**cfg)
    log(f"graph {cfg} {layout} static={static}")
    d = synth.make_inputs(p, DEV)
    fp8 = p.wdtype == "fp8"
    wl = moe.MOE_LAYOUT_TILED if layout == "tiled" else moe.MOE_LAYOUT_ROWS
    if fp8:
        w13, w2, s13, s2 = d.w13q, d.w2q, d.w13s, d.w2s
    else:
        w13, w2, s13, s2 = d.w13, d.w2, None, None
        if layout == "tiled":
            rows = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m)
            w13, w2 = moe.moe_pack_weights(rows, 1, w13), moe.moe_pack_weights(rows, 2, w2)
    wdt = moe.MOE_W_FP8_E4M3_BLOCK128 if fp8 else moe.MOE_W_BF16
    prob = moe.make_problem(p.M, p.H, p.I, p.E, p.topk, p.block_m, wdt, False, wl, 0, p.chunk_tokens)
    ids = torch.empty((p.M, p.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((p.M, p.topk), dtype=torch.float32, device=DEV)
    y = torch.empty((p.M, p.H), dtype=torch.bfloat16, device=DEV)
    ws = None if static else moe.workspace_for(prob, DEV)

    def step(stream=None):
        moe.moe_topk(d.logits, p.topk, out=(ids, w), stream=stream)
        if static:
            moe.fused_experts_static(d.x, w13, w2, ids, w, p.block_m, y, s13, s2, stream=stream,
                                     weight_layout=wl, chunk_tokens=p.chunk_tokens)
        else:
            moe.fused_experts(d.x, w13, w2, ids, w, p.block_m, s13, s2, out=y, workspace=ws, stream=stream,
                              weight_layout=wl, chunk_tokens=p.chunk_tokens)

    step()
    torch.cuda.synchronize()
    ref = y.view(torch.int16).clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device=DEV)
    for i in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref), f"replay {i} differs from the eager call"
        # eager work between the replays, the library's included
        other.mul_(1.0001)
        step()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref), f"eager call after replay {i} differs"
