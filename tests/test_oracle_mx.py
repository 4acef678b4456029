"""Pins for the oracle's MX formats (E8M0 block scales per 32 values; E4M3 and
E2M1 elements).

* Codecs against their bit-field definitions: all 256 E8M0 codes (2^(c-127),
  255 NaN) and all 16 E2M1 codes (1 sign, 2 exponent bits with bias 1, 1
  mantissa bit; exponent 0 is subnormal, m x 0.5); E2M1 rounding on every
  midpoint (ties to the even code) and saturation at 6.
* Quantisation: the scale is the smallest power of two s with amax <= fmax * s
  (checked as amax > fmax * s / 2), the E4M3 codes equal torch's float8 cast of
  v / s, E2M1 codes pack element 2i into the low nibble.
* GEMM: on inputs that the formats hold exactly (grid values times power-of-two
  block scales) the MX GEMM equals the bf16 GEMM bit for bit, for E4M3 and
  E2M1 weights; a transposed scale grid must fail that.
* Layer: close to the bf16 layer on the same master weights (relative RMS).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from hostutil import bf16_f64, bits16


def test_e8m0_codes():
    for c in range(255):
        assert oracle.e8m0_to_f64(c) == math.ldexp(1.0, c - 127)
    assert math.isnan(oracle.e8m0_to_f64(255))


def test_e2m1_codes():
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        got = oracle.e2m1_to_f64(c)
        assert got == (-v if s else v) and math.copysign(1, got) == (-1 if s else 1)


@pytest.mark.parametrize("v,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6),
                                    (5.0, 6), (7.0, 7), (100.0, 7), (0.3, 1), (0.7, 1), (2.9, 5),
                                    (-0.75, 10), (-5.5, 15), (0.0, 0)])
def test_e2m1_rounding(v, code):
    assert oracle.f32_to_e2m1(v) == code


def check_scales(v, sc, fmax):
    amax = np.abs(v.reshape(-1, 32)).max(1).astype(np.float64)
    s = np.ldexp(1.0, sc.reshape(-1).astype(np.int64) - 127)
    nz = amax > 0
    assert np.all(amax[nz] <= fmax * s[nz]) and np.all(amax[nz] > fmax * s[nz] / 2)
    assert np.all(sc.reshape(-1)[~nz] == 0)
    return s


def test_quant_mx_fp8():
    g = np.random.default_rng(0)
    v = (g.standard_normal((6, 256)) * np.exp2(g.integers(-20, 20, (6, 1)))).astype(np.float32)
    v[2, 32:64] = 0.0
    v[3, :32] = 448.0 * 2.0 ** -5     # amax exactly on a power-of-two boundary
    q, sc = oracle.quant_mx_fp8(v)
    s = check_scales(v, sc, 448.0)
    ref = (torch.from_numpy(v.reshape(-1, 32) / s[:, None].astype(np.float32))).to(torch.float8_e4m3fn)
    assert np.array_equal(q.reshape(-1, 32), ref.view(torch.uint8).numpy())
    assert sc[3, 0] == 127 - 5


def test_quant_mx_fp4_packing_and_scale():
    g = np.random.default_rng(1)
    v = (g.standard_normal((4, 128)) * 3).astype(np.float32)
    v[0, :32] = 0.0
    v[0, 32] = 6.0 * 4     # block 1: amax 24 -> scale 4
    v[0, 33] = 0.5 * 4
    q, sc = oracle.quant_mx_fp4(v)
    s = check_scales(v, sc, 6.0)
    assert sc[0, 1] == 127 + 2 and q[0, 16] == (7 | (1 << 4))
    dq = np.array([[oracle.e2m1_to_f64((b >> (4 * h)) & 15) for b in row for h in (0, 1)] for row in q])
    err = np.abs(dq.reshape(-1, 32) * s[:, None] - v.reshape(-1, 32))
    assert np.all(err <= 1.0 * s[:, None] + 1e-12)   # half the widest E2M1 step (2) times s


def grid_problem(fmt, seed):
    """Activations and weights that MX holds exactly: E4M3 (or E2M1) grid values
    times power-of-two block scales."""
    g = np.random.default_rng(seed)
    K, N = 256, 48
    if fmt == "e4m3":
        codes = g.integers(0, 256, (N, K)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x38            # no NaN codes
        wv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    else:
        codes = g.integers(0, 16, (N, K)).astype(np.uint8)
        wv = np.vectorize(oracle.e2m1_to_f64)(codes)
    wsc = g.integers(120, 134, (N, K // 32)).astype(np.uint8)
    w = wv * np.ldexp(1.0, np.repeat(wsc.astype(np.int64) - 127, 32, axis=1))
    acodes = g.integers(0, 256, K).astype(np.uint8)
    acodes[(acodes & 0x7F) == 0x7F] = 0x30
    av = torch.from_numpy(acodes).view(torch.float8_e4m3fn).double().numpy()
    asc = g.integers(122, 131, K // 32).astype(np.uint8)
    a = av * np.ldexp(1.0, np.repeat(asc.astype(np.int64) - 127, 32))
    packed = codes if fmt == "e4m3" else (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return acodes, asc, packed, wsc, a, w


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_gemm_mx_lossless_equals_bf16_gemm(fmt):
    acodes, asc, qw, wsc, a, w = grid_problem(fmt, 3 if fmt == "e4m3" else 4)
    got = oracle.gemm_mx(acodes, asc, qw, wsc, fmt)
    # the same products in bf16: every value here is a bf16 number
    ab = oracle.f64_to_bf16(a).reshape(1, -1)
    wb = oracle.f64_to_bf16(w)
    N, K = w.shape
    ref = oracle.gemm2_bf16(ab[0], wb)      # o[n] = bf16(sum_k a[k] w[n, k])
    assert np.array_equal(got, ref)
    bad = oracle.gemm_mx(acodes, asc, qw, np.ascontiguousarray(wsc[::-1]), fmt)
    assert not np.array_equal(bad, ref)


def test_gemm_w4a8_activation_scales_per_128():
    acodes, _, qw, wsc, a_grid, w = grid_problem("e2m1", 5)
    sa = np.array([0.5, 2.0], np.float32)   # one fp32 scale per 128 columns
    got = oracle.gemm_mx(acodes, sa, qw, wsc, "e2m1")
    av = torch.from_numpy(acodes).view(torch.float8_e4m3fn).double().numpy() * np.repeat(sa, 128)
    ref = oracle.gemm2_bf16(oracle.f64_to_bf16(av), oracle.f64_to_bf16(w))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("w4", [False, True])
def test_mx_layer_close_to_bf16_layer(w4):
    p = synth.Problem(M=16, H=256, I=256, E=4, topk=2, wdtype="w4a8" if w4 else "mxfp8")
    inp = synth.make_inputs(p, "cpu")
    master = synth.make_inputs(synth.Problem(M=16, H=256, I=256, E=4, topk=2), "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), p.topk)
    y = oracle.fused_experts_mx(bits16(inp.x), inp.w13q.view(torch.uint8).numpy(), inp.w13s.numpy(),
                                inp.w2q.view(torch.uint8).numpy(), inp.w2s.numpy(), ids, w, w4=w4)
    y_ref = oracle.fused_experts_bf16(bits16(master.x), bits16(master.w13), bits16(master.w2), ids, w)
    a, b = bf16_f64(y), bf16_f64(y_ref)
    rel = np.sqrt(((a - b) ** 2).mean() / (b ** 2).mean())
    assert rel < (0.25 if w4 else 0.08), rel
    assert rel > 1e-4
