"""Which tokens a full-size parity test checks against the oracle.

At full size the oracle cannot compute every token in test time, so the checked
tokens are chosen from the aligned layout (which the align tests show is the
GPU's, bit for bit) so that every block of block_m rows holds a checked row,
hence every tile of both GEMMs (every column tile of every block, the first and
last tiles of every XCD's range, the split-K tail tiles and the last rounds of
the persistent kernels). A token holds topk rows in different blocks, so the
tokens are picked greedily, each covering the most blocks not yet covered (ties
broken at random, which spreads the checked rows over the 32-row groups of the
blocks): a fraction of one token per block. Added to those: the first and last
tokens, a token of every expert that received exactly one item, and random
tokens up to `at_least`.
"""
from __future__ import annotations

import numpy as np

import oracle


def block_rows(ids: np.ndarray, E: int, block_m: int, expert_map=None, seed: int = 0) -> list[int]:
    """Tokens that together hold a real row of every block of the layout of `ids` [M, k]."""
    M, k = ids.shape
    sorted_ids, _, npp, _ = oracle.align(ids, E, block_m, expert_map=expert_map)
    R = M * k
    item = np.asarray(sorted_ids[:npp], np.int64)
    real = item < R
    blk = np.nonzero(real)[0] // block_m
    tok = item[real] // k
    if blk.size == 0:
        return []
    covered = np.zeros(int(blk.max()) + 1, bool)
    covered[np.setdiff1d(np.arange(covered.size), blk)] = True   # padding-only blocks
    jitter = np.random.default_rng(seed).random(M) * 0.5       # breaks ties only
    toks = []
    while not covered.all():
        open_rows = ~covered[blk]
        gain = np.bincount(tok[open_rows], minlength=M) + jitter
        gain[np.bincount(tok[open_rows], minlength=M) == 0] = -1.0
        t = int(np.argmax(gain))
        toks.append(t)
        covered[blk[tok == t]] = True
    return toks


def pick_tokens(ids: np.ndarray, E: int, block_m: int, expert_map=None, chunk: int = 0,
                at_least: int = 192, at_most: int = 720, seed: int = 0) -> list[int]:
    """Sorted token indices to check. chunk > 0: the layer runs on chunks of that many
    tokens, each with its own layout."""
    M = ids.shape[0]
    rng = np.random.default_rng(seed)
    step = chunk if 0 < chunk < M else M
    blocks = []
    for t0 in range(0, M, step):
        blocks += [t0 + t for t in block_rows(ids[t0:t0 + step], E, block_m, expert_map)]
    if len(blocks) > at_most:   # keep the first and last blocks, thin the middle evenly
        keep = np.unique(np.round(np.linspace(0, len(blocks) - 1, at_most)).astype(int))
        blocks = [blocks[i] for i in keep]
    flat = ids.reshape(-1)
    route = flat if expert_map is None else np.where((flat >= 0) & (flat < len(expert_map)),
                                                     np.asarray(expert_map)[np.clip(flat, 0, len(expert_map) - 1)], -1)
    counts = np.bincount(route[route >= 0], minlength=E)
    singles = [int(np.nonzero(route == e)[0][0]) // ids.shape[1] for e in np.nonzero(counts == 1)[0]]
    toks = set(blocks) | {0, M - 1} | set(singles[:32])
    while len(toks) < min(at_least, M):
        toks.add(int(rng.integers(0, M)))
    return sorted(toks)


def expert_subset(ids: np.ndarray, toks: list[int], E: int):
    """(experts touched by the tokens, ids of those tokens renumbered into that list)."""
    sub = ids[toks]
    experts = sorted(set(int(e) for e in sub.reshape(-1) if 0 <= e < E))
    remap = np.full(E, -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    return experts, remap[sub]
