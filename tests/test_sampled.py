"""The full-size parity tests' token choice covers every block of the layout."""
import numpy as np

import oracle
import sampled
import synth


def test_every_block_holds_a_checked_row():
    p = synth.Problem.named("dsv3_skewed_prefill_m8192")
    small = synth.Problem(M=p.M, H=128, I=128, E=p.E, topk=p.topk, bias_std=p.bias_std)
    ids, _ = oracle.topk(synth.make_inputs(small, "cpu").logits.numpy(), p.topk)
    toks = sampled.pick_tokens(ids, p.E, p.block_m)
    assert len(toks) >= 192
    sorted_ids, _, npp, _ = oracle.align(ids, p.E, p.block_m)
    chosen = np.zeros(p.M, bool)
    chosen[toks] = True
    R = ids.size
    groups = set()
    for b in range(npp // p.block_m):
        rows = sorted_ids[b * p.block_m:(b + 1) * p.block_m]
        real = rows[rows < R]
        hit = chosen[real // p.topk]
        assert hit.any(), f"block {b} has no checked row"
        groups.update((np.nonzero(hit)[0] // 32).tolist())
    assert groups == {0, 1, 2, 3}          # row positions spread over the 32-row groups
    counts = np.bincount(ids.reshape(-1), minlength=p.E)
    for e in np.nonzero(counts == 1)[0]:
        assert chosen[np.nonzero((ids == e).any(1))[0]].any()


def test_chunks_and_small_layouts():
    g = np.random.default_rng(3)
    ids = np.stack([g.choice(8, 2, replace=False) for _ in range(1000)]).astype(np.int32)
    toks = sampled.pick_tokens(ids, 8, 256, chunk=300)
    assert len(toks) >= 128 and toks[0] == 0 and toks[-1] == 999
    for t0 in range(0, 1000, 300):
        sub = ids[t0:t0 + 300]
        s, _, npp, _ = oracle.align(sub, 8, 256)
        chosen = set(t - t0 for t in toks if t0 <= t < t0 + 300)
        for b in range(npp // 256):
            rows = s[b * 256:(b + 1) * 256]
            assert chosen & set((rows[rows < sub.size] // 2).tolist())
