"""Pins for the oracle's number formats (bf16, OCP e4m3fn) and group quantiser.

The oracle's codecs are written from the format definitions; here they are
checked against torch's CPU casts (an independent library routine) over every
bf16 and every e4m3 bit pattern, and against exact tie cases.
"""
import numpy as np
import torch

import oracle
from hostutil import e4m3_f64, from_bits16


def test_bf16_decode_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f64(pats)
    ref = from_bits16(pats).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_bf16_encode_matches_torch_on_fp32_values():
    # every double that is exactly an fp32 value rounds once, so torch's
    # fp32 -> bf16 cast (RNE) is an exact reference
    g = np.random.default_rng(1)
    bits = g.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    mine = oracle.f64_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_encode_ties_to_even():
    # midpoints between neighbouring positive finite bf16 numbers are exact in fp64
    lo = np.arange(0x0000, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    hi = lo + 1
    lo_v = oracle.bf16_to_f64(lo)
    hi_v = oracle.bf16_to_f64(hi)
    mid = (lo_v + hi_v) / 2
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(oracle.f64_to_bf16(mid), even)
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, np.inf)), hi)
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, -np.inf)), lo)
    # sign symmetry
    assert np.array_equal(oracle.f64_to_bf16(-mid), even | 0x8000)


def test_bf16_encode_overflow_and_zero():
    big = oracle.bf16_to_f64(np.array([0x7F7F], np.uint16))[0]
    half_ulp = 2.0 ** (127 - 8)
    assert oracle.f64_to_bf16(np.array([big + half_ulp * 0.99]))[0] == 0x7F7F
    assert oracle.f64_to_bf16(np.array([big + half_ulp]))[0] == 0x7F80
    assert oracle.f64_to_bf16(np.array([-0.0]))[0] == 0x8000
    assert oracle.f64_to_bf16(np.array([0.0]))[0] == 0x0000


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = e4m3_f64(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(2)
    v = np.concatenate([
        g.uniform(-448, 448, 200_000),
        g.standard_normal(100_000) * 2.0 ** g.integers(-12, 8, 100_000),
    ]).astype(np.float32)
    v = np.clip(v, -448, 448)
    mine = oracle.f32_to_e4m3(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encode_ties_to_even_and_saturation():
    codes = np.arange(0x00, 0x7E, dtype=np.uint8)          # 0 .. 416 (0x7D), pairs (c, c+1)
    lo_v = oracle.e4m3_to_f64(codes)
    hi_v = oracle.e4m3_to_f64(codes + 1)
    mid = ((lo_v + hi_v) / 2).astype(np.float32)          # exact in fp32
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(oracle.f32_to_e4m3(mid), even)
    assert np.array_equal(oracle.f32_to_e4m3(np.nextafter(mid, np.float32(np.inf))), codes + 1)
    assert np.array_equal(oracle.f32_to_e4m3(np.nextafter(mid, np.float32(-np.inf))), codes)
    assert oracle.f32_to_e4m3(np.array([1000.0], np.float32))[0] == 0x7E
    assert oracle.f32_to_e4m3(np.array([-1000.0], np.float32))[0] == 0xFE


def test_quant_groups_definition():
    g = np.random.default_rng(3)
    v = (g.standard_normal((5, 512)) * 2.0 ** g.integers(-6, 6, (5, 1))).astype(np.float32)
    v[2, 128:256] = 0.0                                     # an all-zero group
    q, s = oracle.quant_groups_fp8(v)
    vt = torch.from_numpy(v).view(5, 4, 128)
    amax = vt.abs().amax(-1)
    s_ref = amax / 448.0
    assert np.array_equal(s, s_ref.numpy())
    assert s[2, 1] == 0.0 and np.all(q[2, 128:256] == 0)
    safe = torch.where(s_ref > 0, s_ref, torch.ones_like(s_ref))
    q_ref = (vt / safe[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    q_ref = q_ref.view(torch.uint8).view(5, 512).numpy()
    assert np.array_equal(q, q_ref)
    # the group maximum maps to the top code
    for r in range(5):
        for gi in range(4):
            if s[r, gi] > 0:
                assert np.max(q[r, gi * 128:(gi + 1) * 128] & 0x7F) == 0x7E
