"""Seeded synthetic inputs for the fused MoE expert forward.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``mixture_experts_ffn_block_amd``). It only draws random numbers and stores
them in the dtypes the path consumes; it computes none of the layer's
arithmetic (no routing, no GEMM, no activation, no reduction).

The one encoding it performs is the offline 128x128 block quantisation of the
fp8 weights. On the pages this happens when the checkpoint is loaded, before
any forward runs ("DeepGEMM FusedMoE on Blackwell", section 2.8(c), weight
pre-processing). It is done here with torch's own float8_e4m3fn cast, so both
sides receive the same weight bytes and scales.

Recipe (every tensor is drawn from its own generator, seeded by
``(seed, tensor id, expert)``, so the values do not depend on how the
generation is chunked):

* ``x``       [M, H]  ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even).
* ``logits``  [M, E]  ~ N(0, 1) fp32, plus a per-expert bias ~ N(0, bias_std)
  when the workload asks for skewed routing.
* ``score_bias`` [E] ~ N(0, score_bias_std) fp32: the router's correction bias
  (grouped sigmoid routing), when the workload has one.
* ``w13``     [E, 2I, H] ~ N(0, 1/sqrt(H)) -> bf16; rows [0, I) are the gate
  projection, rows [I, 2I) the up projection.
* ``w2``      [E, H, I]  ~ N(0, 1/sqrt(I)) -> bf16.
* fp8 workloads: ``w13q``/``w2q`` float8_e4m3fn with fp32 scales per 128x128
  block, ``scale = amax(block) / 448``, ``q = e4m3(w / scale)``.
* MX workloads (offline weight preparation as well, [DG] TL;DR: MXFP8 1x32 and
  W4A8 MXFP4): ``wdtype="mxfp8"`` gives E4M3 weights and ``"w4a8"`` E2M1 weights
  (two per byte, element 2i in the low nibble), each 32 columns of a row
  sharing one E8M0 scale 2^ceil(log2(amax / fmax)) (fmax 448 or 6), stored
  [E, N, K/32] uint8; E2M1 takes the nearest grid value (ties to the smaller).
* Spread scales (``scale_spread`` = s > 0, quantised formats only): before
  quantisation every bf16 master is multiplied by powers of two, so that the
  block scales differ by up to 2^(2s+4) inside a tensor and a scale read from
  the wrong block, group or expert changes the result by a large factor. Weight
  blocks (one per 128 rows x 128 columns for fp8, x 32 columns for the MX
  formats) get 2^(c_e + d) with c_e ~ U{-2..2} per expert and d ~ U{-s..s} per
  block; x gets 2^d per (token, 128 columns) (fp8, W4A8) or (token, 32
  columns) (MXFP8). Each factor table has its own seeded generator.
* Expert-parallel workloads (``ep_size`` > 1): the logits cover all E experts
  (global routing); rank ``ep_rank`` holds the contiguous range of E / ep_size
  experts starting at ``ep_rank * E / ep_size``, whose weights are the same
  draws as in the unsharded workload, and ``expert_map`` [E] int32 sends a
  global expert to its index in that range or to -1.

The second argument of N(.,.) is the standard deviation.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

# Named workloads. Sizes and routing statistics follow the pages' usual model
# shapes; block_m is the row-block size shared by the align step and the GEMMs.
WORKLOADS = {
    "tiny": dict(M=64, H=256, I=512, E=8, topk=2, wdtype="bf16", block_m=16, bias_std=0.0),
    # block_m 128: 3 % padded rows against 12 % with 256-row blocks (GEMM1 2 % faster)
    "mixtral_prefill_m4096": dict(M=4096, H=4096, I=14336, E=8, topk=2, wdtype="bf16",
                                  block_m=128, bias_std=0.0),
    "dsv3_skewed_prefill_m8192": dict(M=8192, H=7168, I=2048, E=256, topk=8, wdtype="bf16",
                                      block_m=128, bias_std=1.5),
    "decode_m32": dict(M=32, H=2048, I=768, E=128, topk=8, wdtype="bf16", block_m=16,
                       bias_std=0.0),
    "fp8_block_m4096": dict(M=4096, H=7168, I=2048, E=256, topk=8, wdtype="fp8",
                            block_m=128, bias_std=0.0),
    # the fp8 workload's shapes and routing in MXFP8 (E8M0 scale per 32 values)
    "mxfp8_m4096": dict(M=4096, H=7168, I=2048, E=256, topk=8, wdtype="mxfp8", block_m=128),
    # the same in W4A8: E2M1 weights with E8M0 scales per 32, fp8 activations per 128
    "w4a8_m4096": dict(M=4096, H=7168, I=2048, E=256, topk=8, wdtype="w4a8", block_m=128),
    # a long prefill on the Mixtral shape, run in two chunks of 16K tokens
    "mixtral_prefill_m32768_chunk16k": dict(M=32768, H=4096, I=14336, E=8, topk=2, wdtype="bf16",
                                            block_m=256, chunk_tokens=16384),
    # DeepSeek-V3-style routing on the DSV3 shape: sigmoid scores, 8 groups of 32
    # experts of which 4 are kept, a correction bias, weights scaled by 2.5
    "dsv3_grouped_prefill_m8192": dict(M=8192, H=7168, I=2048, E=256, topk=8, wdtype="bf16",
                                       block_m=128, scoring="sigmoid", n_group=8, topk_group=4,
                                       score_bias_std=0.05, routed_scale=2.5),
    # the decode routing presented in the batched-experts form: one batch of up to
    # M rows per expert (a token sends at most one item to an expert)
    "decode_batched_m32": dict(M=32, H=2048, I=768, E=128, topk=8, wdtype="bf16", block_m=16,
                               bias_std=0.0, batched=True),
    # one rank of an 8-way expert-parallel split of the skewed workload: the rank
    # with the most routed items (13863 of 65536, 20 experts touched) when the
    # inputs are drawn on the GPU (torch's CPU and GPU generators differ), which
    # sets the step time of the split layer
    "dsv3_ep8_rank2_prefill_m8192": dict(M=8192, H=7168, I=2048, E=256, topk=8, wdtype="bf16",
                                         block_m=128, bias_std=1.5, ep_size=8, ep_rank=2),
}

_T_X, _T_LOGITS, _T_BIAS, _T_W13, _T_W2, _T_SCORE_BIAS = 1, 2, 3, 4, 5, 6
_T_SPREAD_X, _T_SPREAD_W13, _T_SPREAD_W2 = 7, 8, 9


@dataclasses.dataclass
class Problem:
    """Sizes and options of one fused MoE call."""

    M: int
    H: int
    I: int
    E: int
    topk: int
    wdtype: str = "bf16"          # "bf16" or "fp8" (e4m3 weights + 128x128 fp32 scales)
    block_m: int = 16
    bias_std: float = 0.0
    seed: int = 0
    apply_router_weight_on_input: bool = False
    ep_size: int = 1              # expert-parallel ranks; E counts the global experts
    ep_rank: int = 0
    batched: bool = False         # the expert layer takes the batched-experts form
    # router: scoring "softmax" or "sigmoid", groups (1 = none), kept groups, the
    # correction bias's standard deviation (0 = none), the routed scaling factor
    scoring: str = "softmax"
    n_group: int = 1
    topk_group: int = 1
    score_bias_std: float = 0.0
    routed_scale: float = 1.0
    chunk_tokens: int = 0         # > 0: the layer runs on chunks of this many tokens
    scale_spread: int = 0         # > 0: power-of-two factors spread the quantisation scales

    @property
    def local_experts(self) -> range:
        """Global ids of the experts this rank holds (all E without expert parallelism)."""
        n = self.E // self.ep_size
        return range(self.ep_rank * n, (self.ep_rank + 1) * n)

    @staticmethod
    def named(name: str, **overrides) -> "Problem":
        d = dict(WORKLOADS[name])
        d.update(overrides)
        return Problem(**d)


def _gen(device, seed: int, tensor_id: int, expert: int = 0) -> torch.Generator:
    # torch's CPU generator keeps only the low 32 bits of a seed, so the tuple
    # is hashed down to 32 bits rather than packed into a wider integer
    h = hashlib.blake2b(f"{seed}/{tensor_id}/{expert}".encode(), digest_size=4).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h, "little"))
    return g


def _randn(shape, device, seed, tensor_id, expert=0, std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed, tensor_id, expert),
                    dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t


def _spread_rows(n_rows: int, n_cols: int, col_block: int, device, seed, tensor_id, expert,
                 spread: int, per_expert: bool) -> torch.Tensor:
    """fp32 factors 2^p [n_rows, n_cols]: one exponent per 128 rows x col_block columns
    (per row x col_block columns when not per_expert, for activations), p = c + d with
    c ~ U{-2..2} for the expert (0 for activations) and d ~ U{-spread..spread}."""
    g = _gen(device, seed, tensor_id, expert)
    rb = 128 if per_expert else 1
    c = int(torch.randint(-2, 3, (1,), generator=g, device=device).item()) if per_expert else 0
    d = torch.randint(-spread, spread + 1, (n_rows // rb, n_cols // col_block), generator=g, device=device)
    f = torch.exp2((c + d).float())
    return f.repeat_interleave(rb, 0).repeat_interleave(col_block, 1)


def block_quant_fp8(w: torch.Tensor):
    """128x128 block quantisation of a bf16 [N, K] matrix (offline weight prep).

    Returns (q float8_e4m3fn [N, K], scale fp32 [N/128, K/128]).
    """
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    wf = w.float().view(N // 128, 128, K // 128, 128)
    amax = wf.abs().amax(dim=(1, 3))                       # [N/128, K/128]
    scale = amax / 448.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    # an all-zero block keeps scale 0 and divides by 1, giving zero codes
    q = (wf / safe[:, None, :, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(N, K), scale


_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_MX_STACK = 1 << 27  # weights quantised per mx_quant call when MX weights are drawn


def mx_quant(w: torch.Tensor, fmt: str):
    """1x32 MX quantisation of a bf16 [N, K] matrix (offline weight prep).

    Returns (codes, scales): E4M3 float8_e4m3fn [N, K] or packed E2M1 uint8 [N, K/2],
    and E8M0 codes uint8 [N, K/32].
    """
    N, K = w.shape
    wf = w.float().view(N, K // 32, 32)
    amax = wf.abs().amax(-1)
    fmax = 448.0 if fmt == "e4m3" else 6.0
    safe = torch.where(amax > 0, amax, torch.full_like(amax, fmax))
    e = torch.ceil(torch.log2(safe / fmax)).clamp_(-127, 127)
    e = torch.where(amax > 0, e, torch.full_like(e, -127))
    v = wf / torch.exp2(e)[..., None]
    sc = (e + 127).to(torch.uint8)
    if fmt == "e4m3":
        return v.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(N, K), sc
    mags = torch.tensor(_E2M1, device=w.device)
    idx = (v.abs().clamp(max=6.0)[..., None] - mags).abs().argmin(-1).to(torch.uint8)
    codes = (idx | (v < 0).to(torch.uint8) << 3).view(N, K)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous(), sc


@dataclasses.dataclass
class Inputs:
    x: torch.Tensor                   # [M, H] bf16
    logits: torch.Tensor              # [M, E] fp32
    w13: torch.Tensor | None          # [E, 2I, H] bf16 (bf16 workloads)
    w2: torch.Tensor | None           # [E, H, I] bf16
    w13q: torch.Tensor | None = None  # [E, 2I, H] float8_e4m3fn (fp8, mxfp8), [E, 2I, H/2] uint8 (w4a8)
    w13s: torch.Tensor | None = None  # [E, 2I/128, H/128] fp32 (fp8), [E, 2I, H/32] uint8 E8M0 (MX)
    w2q: torch.Tensor | None = None   # [E, H, I] float8_e4m3fn
    w2s: torch.Tensor | None = None   # [E, H/128, I/128] fp32
    expert_map: torch.Tensor | None = None  # [E] int32 on expert-parallel ranks, else None
    score_bias: torch.Tensor | None = None  # [E] fp32 router correction bias, else None


def make_inputs(p: Problem, device="cpu") -> Inputs:
    """Draw the seeded synthetic inputs of problem ``p`` on ``device``."""
    M, H, I, E = p.M, p.H, p.I, p.E
    spread = p.scale_spread if p.wdtype != "bf16" else 0
    kb = 32 if p.wdtype in ("mxfp8", "w4a8") else 128   # columns per weight scale block
    x = _randn((M, H), device, p.seed, _T_X)
    if spread and M:
        x *= _spread_rows(M, H, 32 if p.wdtype == "mxfp8" else 128, device, p.seed, _T_SPREAD_X, 0,
                          spread, False)
    x = x.to(torch.bfloat16)

    def master13(e):
        m = _randn((2 * I, H), device, p.seed, _T_W13, e, 1.0 / math.sqrt(H))
        if spread:
            m *= _spread_rows(2 * I, H, kb, device, p.seed, _T_SPREAD_W13, e, spread, True)
        return m.to(torch.bfloat16)

    def master2(e):
        m = _randn((H, I), device, p.seed, _T_W2, e, 1.0 / math.sqrt(I))
        if spread:
            m *= _spread_rows(H, I, kb, device, p.seed, _T_SPREAD_W2, e, spread, True)
        return m.to(torch.bfloat16)

    logits = _randn((M, E), device, p.seed, _T_LOGITS)
    if p.bias_std:
        logits += _randn((E,), device, p.seed, _T_BIAS, std=p.bias_std)[None, :]
    sbias = _randn((E,), device, p.seed, _T_SCORE_BIAS, std=p.score_bias_std) if p.score_bias_std else None
    held = p.local_experts
    emap = None
    if p.ep_size > 1:
        emap = torch.full((E,), -1, dtype=torch.int32)
        emap[held.start:held.stop] = torch.arange(len(held), dtype=torch.int32)
        emap = emap.to(device)
    EL = len(held)
    if p.wdtype == "bf16":
        w13 = torch.empty((EL, 2 * I, H), dtype=torch.bfloat16, device=device)
        w2 = torch.empty((EL, H, I), dtype=torch.bfloat16, device=device)
        for i, e in enumerate(held):
            w13[i] = _randn((2 * I, H), device, p.seed, _T_W13, e, 1.0 / math.sqrt(H))
            w2[i] = _randn((H, I), device, p.seed, _T_W2, e, 1.0 / math.sqrt(I))
        return Inputs(x, logits, w13, w2, expert_map=emap, score_bias=sbias)
    if p.wdtype == "fp8":
        w13q = torch.empty((EL, 2 * I, H), dtype=torch.float8_e4m3fn, device=device)
        w2q = torch.empty((EL, H, I), dtype=torch.float8_e4m3fn, device=device)
        w13s = torch.empty((EL, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        w2s = torch.empty((EL, H // 128, I // 128), dtype=torch.float32, device=device)
        for i, e in enumerate(held):
            w13q[i], w13s[i] = block_quant_fp8(master13(e))
            w2q[i], w2s[i] = block_quant_fp8(master2(e))
        return Inputs(x, logits, None, None, w13q, w13s, w2q, w2s, expert_map=emap, score_bias=sbias)
    if p.wdtype in ("mxfp8", "w4a8"):
        fmt = "e4m3" if p.wdtype == "mxfp8" else "e2m1"
        div = 1 if fmt == "e4m3" else 2
        dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.uint8
        w13q = torch.empty((EL, 2 * I, H // div), dtype=dt, device=device)
        w2q = torch.empty((EL, H, I // div), dtype=dt, device=device)
        w13s = torch.empty((EL, 2 * I, H // 32), dtype=torch.uint8, device=device)
        w2s = torch.empty((EL, H, I // 32), dtype=torch.uint8, device=device)
        # the quantiser works row by row, so a stack of experts gets each expert's own
        # codes and scales; stacks of up to _MX_STACK weights make far fewer launches
        step = max(1, _MX_STACK // (2 * I * H))
        experts = list(held)
        for j in range(0, EL, step):
            stack = experts[j:j + step]
            n = len(stack)
            m13 = torch.stack([master13(e) for e in stack])
            q, sc = mx_quant(m13.view(n * 2 * I, H), fmt)
            w13q[j:j + n], w13s[j:j + n] = q.view(n, 2 * I, -1), sc.view(n, 2 * I, -1)
            m2 = torch.stack([master2(e) for e in stack])
            q, sc = mx_quant(m2.view(n * H, I), fmt)
            w2q[j:j + n], w2s[j:j + n] = q.view(n, H, -1), sc.view(n, H, -1)
        return Inputs(x, logits, None, None, w13q, w13s, w2q, w2s, expert_map=emap, score_bias=sbias)
    raise ValueError(f"unknown weight dtype {p.wdtype!r}")

