"""Exact float64 reference and a derived per-element error bound for the 8-bit layers.

The reference is the layer's formula ("fused_moe.py analysis", 1.1-1.2; "DeepGEMM
FusedMoE on Blackwell", 1.1) evaluated in float64 on the dequantised weights, with
the activations x and z NOT quantised:

    y_t = sum_j a2_j W2_e (a1_j SiLU(G_e x_t) * (U_e x_t))     (a1, a2 = alpha, 1 or 1, alpha)

A correct 8-bit implementation differs from it only by its roundings: x and z
quantised to e4m3 (per 128 columns with an fp32 scale amax/448, or per 32 with an
E8M0 scale), h, o and y rounded to bf16, the fp32 product alpha*SiLU(g)*u, and
the accumulation error of the sums. Each rounding is bounded on its own and the
bounds are carried through the layer with absolute values:

* e4m3 (3 stored mantissa bits, subnormal spacing 2^-9): a value v coded against
  a scale s is off by at most 2^-4 |v| + 2^-10 s, plus 2^-21 |v| for the fp32
  division and the clamp at 448. For the fp32 scale s <= amax / 448 (1 + 2^-23);
  for E8M0, s < 2 amax / 448.
* bf16 (8 significant bits): one rounding moves a value by at most 2^-9 of itself.
* SiLU is 1.1-Lipschitz (|SiLU'| <= 1.0999) and |SiLU(g)| <= |g|.
* a sum of n products accumulated in precision u is off by at most n u times the
  sum of their magnitudes (``acc_eps`` per term: ~2^-52 K for the fp64 oracle,
  2^-23 K for an fp32 GEMM).

A mistake that mixes up scales (another expert's, another block's, a transposed
grid) changes values by whole powers of two when the scales are spread
(``synth.Problem.scale_spread``), which the bound does not allow. The bound is
worst case over the signs of the errors, so it is loose (typically 10-50x the
actual error), and the tests check that it is not vacuous.
"""
from __future__ import annotations

import numpy as np
import torch

U4 = 2.0 ** -4    # e4m3 half-ulp, relative
SUB = 2.0 ** -10  # e4m3 half subnormal spacing, in units of the scale
BF = 2.0 ** -9    # bf16 half-ulp, relative
DIVF = 2.0 ** -21


def e4m3(a) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().numpy()


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_packed(a: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] (element 2i in the low nibble) -> float64 [..., K]."""
    lo, hi = a & 15, a >> 4
    both = np.stack([lo, hi], -1).reshape(a.shape[:-1] + (a.shape[-1] * 2,))
    mag = E2M1[both & 7]
    return np.where(both & 8, -mag, mag)


def deq_fp8_block(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """e4m3 codes [E, N, K] with fp32 scales [E, N/128, K/128] -> float64 [E, N, K]."""
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)
    return e4m3(q) * sc


def deq_mx(q: np.ndarray, codes: np.ndarray, fp4: bool) -> np.ndarray:
    """E4M3 [E, N, K] or packed E2M1 [E, N, K/2] with E8M0 codes [E, N, K/32] -> float64."""
    v = e2m1_packed(q) if fp4 else e4m3(q)
    return v * np.repeat(np.exp2(codes.astype(np.float64) - 127.0), 32, -1)


def quant_err(vabs: np.ndarray, group: int, e8m0: bool) -> np.ndarray:
    """Bound on |dequant(quant(v)) - v| for values with |v| <= vabs (last axis grouped)."""
    shp = vabs.shape
    g = vabs.reshape(shp[:-1] + (shp[-1] // group, group))
    amax = g.max(-1, keepdims=True)
    s = amax / 448.0 * (2.0 if e8m0 else 1.0 + 2.0 ** -22)
    return ((U4 + DIVF) * g + SUB * s).reshape(shp)


def silu(g):
    with np.errstate(over="ignore"):   # exp(-g) = inf for very negative g: SiLU(g) = -0
        return g / (1.0 + np.exp(-g))


class Act:
    """How x and z are quantised: group width and scale type."""

    def __init__(self, group: int, e8m0: bool):
        self.group, self.e8m0 = group, e8m0


FP8_128 = Act(128, False)   # fp8 block and W4A8: fp32 scale per 128
MX_32 = Act(32, True)       # MXFP8: E8M0 scale per 32


def slot_bound(x: np.ndarray, W13: np.ndarray, W2: np.ndarray, a1: float, act: Act, acc_eps1: float,
               acc_eps2: float):
    """One token through one expert: (o_exact [H], bound on |o - o_exact| [H], |o| bound)."""
    I = W13.shape[0] // 2
    ax = np.abs(x)
    ex = quant_err(ax, act.group, act.e8m0)
    aW13 = np.abs(W13)
    h = W13 @ x
    eh = aW13 @ ex + acc_eps1 * (aW13 @ (ax + ex))
    eh = eh + BF * (np.abs(h) + eh)
    g, u, eg, eu = h[:I], h[I:], eh[:I], eh[I:]
    sg = silu(g)
    z = a1 * sg * u
    ezf = a1 * (1.1 * eg * (np.abs(u) + eu) + np.abs(sg) * eu)
    zmag = np.abs(z) + ezf
    ezf = ezf + 2.0 ** -19 * zmag          # fp32 SiLU (exp approximation, divide) and product
    zmag = np.abs(z) + ezf
    ez = ezf + quant_err(zmag, act.group, act.e8m0)
    aW2 = np.abs(W2)
    o = W2 @ z
    eo = aW2 @ ez + acc_eps2 * (aW2 @ (zmag + ez))
    eo = eo + BF * (np.abs(o) + eo)
    return o, eo


def layer_reference(x: np.ndarray, ids: np.ndarray, w: np.ndarray, W13: np.ndarray, W2: np.ndarray,
                    act: Act, on_input: bool = False, fp32_acc: bool = False, expert_map=None):
    """(y_exact [M, H], bound [M, H]) for the routed layer. W13 / W2 are the dequantised
    weights [E, 2I, H] / [E, H, I] of the experts held (expert_map: global -> local or -1).
    fp32_acc: the GEMM sums are fp32 (a GPU kernel), else fp64 (the oracle)."""
    M, H = x.shape
    I = W13.shape[1] // 2
    eps1 = (H * 2.0 ** -23) if fp32_acc else (H * 2.0 ** -52)
    eps2 = (I * 2.0 ** -23) if fp32_acc else (I * 2.0 ** -52)
    y = np.zeros((M, H))
    b = np.zeros((M, H))
    for t in range(M):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if expert_map is not None:
                e = int(expert_map[e]) if 0 <= e < len(expert_map) else -1
                if e < 0:
                    continue
            a = float(w[t, j])
            o, eo = slot_bound(x[t], W13[e], W2[e], a if on_input else 1.0, act, eps1, eps2)
            a2 = 1.0 if on_input else a
            y[t] += a2 * o
            b[t] += abs(a2) * eo
        b[t] = b[t] + 1e-15 * np.abs(y[t]) + BF * (np.abs(y[t]) + b[t])
    return y, b


def batched_reference(a: np.ndarray, counts: np.ndarray, W13: np.ndarray, W2: np.ndarray, act: Act,
                      fp32_acc: bool = False):
    """(out_exact [E, max_M, H], bound) of the batched form: rows past a count are exactly 0."""
    E, max_M, H = a.shape
    I = W13.shape[1] // 2
    eps1 = (H * 2.0 ** -23) if fp32_acc else (H * 2.0 ** -52)
    eps2 = (I * 2.0 ** -23) if fp32_acc else (I * 2.0 ** -52)
    out = np.zeros((E, max_M, H))
    b = np.zeros((E, max_M, H))
    for e in range(E):
        for i in range(min(max(int(counts[e]), 0), max_M)):
            out[e, i], b[e, i] = slot_bound(a[e, i], W13[e], W2[e], 1.0, act, eps1, eps2)
    return out, b


def check(y: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str) -> float:
    """Assert |y - ref| <= bound everywhere; returns the largest err / bound."""
    err = np.abs(y - ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} of {err.size} elements outside the derived bound, "
                           f"first {bad[:4].tolist()}, worst err/bound {(err / bound).max():.3g}")
    return float((err / np.maximum(bound, 1e-300)).max())


def violates(y: np.ndarray, ref: np.ndarray, bound: np.ndarray) -> bool:
    return bool(np.any(np.abs(y - ref) > bound))
