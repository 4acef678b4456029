"""Grouped / sigmoid router on the GPU against the oracle: ids bit for bit,
weights within 1e-6 (times the routed scaling factor)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_block_amd as moe
import oracle
from test_gpu_parity import DEV, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


CASES = [
    # DeepSeek-V3-like: 256 experts in 8 groups, keep 4, top-8, sigmoid + correction bias, x2.5
    dict(M=8192, E=256, k=8, scoring="sigmoid", G=8, TG=4, bias=0.05, scale=2.5, renorm=True),
    dict(M=1000, E=160, k=6, scoring="softmax", G=8, TG=3, bias=None, scale=1.0, renorm=True),
    dict(M=500, E=160, k=6, scoring="softmax", G=8, TG=3, bias=None, scale=1.0, renorm=False),
    dict(M=700, E=128, k=8, scoring="sigmoid", G=1, TG=1, bias=None, scale=1.0, renorm=False),
    dict(M=700, E=128, k=8, scoring="sigmoid", G=1, TG=1, bias=0.3, scale=1.5, renorm=True),
    dict(M=300, E=64, k=8, scoring="sigmoid", G=64, TG=32, bias=None, scale=1.0, renorm=True),
    dict(M=300, E=96, k=4, scoring="sigmoid", G=32, TG=2, bias=1.0, scale=1.0, renorm=True),
    dict(M=33, E=16, k=3, scoring="sigmoid", G=4, TG=2, bias=0.1, scale=2.0, renorm=False),
]
CASE_ID = lambda c: "-".join(f"{k}{v}" for k, v in c.items())


def check(logits, c, bias):
    ids, w = moe.moe_topk_grouped(logits.to(DEV), c["k"], c["scoring"], c["renorm"], c["G"], c["TG"],
                                  None if bias is None else bias.to(DEV), c["scale"])
    rids, rw = oracle.topk_grouped(logits.numpy(), c["k"], c["scoring"], c["renorm"], c["G"], c["TG"],
                                   None if bias is None else bias.numpy(), c["scale"])
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6 * max(1.0, c["scale"])


@pytest.mark.parametrize("c", CASES, ids=CASE_ID)
def test_grouped_router_matches_oracle(c):
    log(f"grouped router {c}")
    g = torch.Generator().manual_seed(c["M"] + c["E"])
    logits = torch.randn((c["M"], c["E"]), generator=g)
    bias = None if c["bias"] is None else torch.randn(c["E"], generator=g) * c["bias"]
    check(logits, c, bias)


def test_grouped_router_worked_example_and_ties():
    # the oracle's hand-worked example: keys 0.5 + bias, groups of two
    b = torch.tensor([0.1, 0.2, 0.0, 0.0, 0.3, -0.5, 0.05, 0.05])
    c = dict(k=3, scoring="sigmoid", renorm=False, G=4, TG=2, scale=1.0)
    ids, w = moe.moe_topk_grouped(torch.zeros((5, 8), device=DEV), 3, "sigmoid", False, 4, 2, b.to(DEV))
    assert ids.cpu().tolist() == [[1, 0, 6]] * 5 and w.cpu().tolist() == [[0.5, 0.5, 0.5]] * 5
    check(torch.zeros((5, 8)), c, b)
    # equal logits everywhere: lowest groups and lowest experts win
    check(torch.zeros((7, 64)), dict(k=4, scoring="softmax", renorm=True, G=8, TG=2, scale=1.0), None)
