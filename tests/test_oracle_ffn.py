"""Pins for the oracle's expert FFN and the whole layer (bf16 and fp8).

* Each step (GEMM1, SiLU-and-mul, GEMM2, block-scaled fp8 GEMM) is compared
  with numpy float64 on the same decoded values: one round-to-nearest-even
  step may move a value by at most 2^-8 of itself.
* Layer invariants: the routed form equals the dense all-experts form; weight
  on the input equals weight on the output (exactly, for power-of-two weights);
  scaling w2 by 2 scales y by exactly 2; zero inputs give zero outputs.
* fp8: on inputs that quantise losslessly the fp8 GEMM equals the bf16 GEMM
  bit for bit, which pins the scale indexing.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hostutil import bf16_f64, bits16, bits8, e4m3_f64

RNE = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits): one RNE step moves a value by at most this fraction


def silu(g):
    return g / (1.0 + np.exp(-g))


def small_problem(M=6, H=256, I=128, E=4, k=2, seed=0):
    p = synth.Problem(M=M, H=H, I=I, E=E, topk=k, seed=seed)
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), k)
    return p, bits16(inp.x), bits16(inp.w13), bits16(inp.w2), ids, w


def test_gemm1_and_act_and_gemm2_against_numpy():
    _, x, w13, w2, _, _ = small_problem()
    xf, w13f, w2f = bf16_f64(x), bf16_f64(w13), bf16_f64(w2)
    for t in range(3):
        for e in range(2):
            h = oracle.gemm1_bf16(x[t], w13[e])
            h64 = w13f[e] @ xf[t]
            assert np.all(np.abs(bf16_f64(h) - h64) <= RNE * np.abs(h64) + 1e-300)
            hf = bf16_f64(h)
            I = hf.size // 2
            for alpha in (1.0, 0.3):
                z = oracle.act_bf16(h, alpha)
                z64 = alpha * silu(hf[:I]) * hf[I:]
                assert np.all(np.abs(bf16_f64(z) - z64) <= RNE * np.abs(z64) + 1e-300)
            z = oracle.act_bf16(h)
            o = oracle.gemm2_bf16(z, w2[e])
            o64 = w2f[e] @ bf16_f64(z)
            assert np.all(np.abs(bf16_f64(o) - o64) <= RNE * np.abs(o64) + 1e-300)


def test_single_expert_is_textbook_swiglu():
    # E = 1, k = 1, weight 1: the layer is W2 (SiLU(G x) * (U x))
    p, x, w13, w2, _, _ = small_problem(M=8, E=1, k=1)
    ids = np.zeros((8, 1), np.int32)
    w = np.ones((8, 1), np.float32)
    y = oracle.fused_experts_bf16(x, w13, w2, ids, w)
    xf, w13f, w2f = bf16_f64(x), bf16_f64(w13)[0], bf16_f64(w2)[0]
    I = p.I
    g, u = w13f[:I] @ xf.T, w13f[I:] @ xf.T
    ref = (w2f @ (silu(g) * u)).T                                  # float64, no rounding
    # error bound: rounding g, u (h) and z moves each z_i by at most ~3.1 RNE
    # of |g_i u_i| (|SiLU'| <= 1.1, |SiLU(g)| <= |g|); W2 carries that into y;
    # o and y add one rounding each
    bound = 3.2 * RNE * (np.abs(w2f) @ np.abs(g * u)).T + 2.1 * RNE * np.abs(ref)
    err = np.abs(bf16_f64(y) - ref)
    assert np.all(err <= bound), (err / bound).max()
    assert (err / bound).max() > 0.01      # the bound is not vacuous


def test_routed_equals_dense():
    _, x, w13, w2, ids, w = small_problem(M=10, E=6, k=3, seed=4)
    y, acc = oracle.fused_experts_bf16(x, w13, w2, ids, w, return_acc=True)
    yd, accd = oracle.dense_experts_bf16(x, w13, w2, ids, w, return_acc=True)
    np.testing.assert_allclose(acc, accd, rtol=1e-12, atol=1e-300)
    ulp = np.abs(bf16_f64(y) - bf16_f64(yd)) / np.maximum(np.abs(bf16_f64(yd)), 1e-30)
    assert np.all(ulp <= 2.0 ** -7)


def test_router_weight_on_input_equals_on_output():
    _, x, w13, w2, ids, _ = small_problem(M=8, E=4, k=2, seed=5)
    w = np.tile(np.array([0.5, 0.25], np.float32), (8, 1))      # powers of two: exact
    y_out = oracle.fused_experts_bf16(x, w13, w2, ids, w, on_input=False)
    y_in = oracle.fused_experts_bf16(x, w13, w2, ids, w, on_input=True)
    assert np.array_equal(y_in, y_out)
    # general weights: equal up to bf16 rounding at z and o
    _, _, _, _, ids, w = small_problem(M=8, E=4, k=2, seed=6)
    a = bf16_f64(oracle.fused_experts_bf16(x, w13, w2, ids, w, on_input=False))
    b = bf16_f64(oracle.fused_experts_bf16(x, w13, w2, ids, w, on_input=True))
    assert np.all(np.abs(a - b) <= 2e-2 * np.maximum(1.0, np.abs(a)))


def test_scaling_w2_by_two_scales_y_exactly():
    _, x, w13, w2, ids, w = small_problem(M=6, seed=7)
    w2x2 = bits16(torch.from_numpy(bf16_f64(w2) * 2.0).to(torch.bfloat16))
    y1 = oracle.fused_experts_bf16(x, w13, w2, ids, w)
    y2 = oracle.fused_experts_bf16(x, w13, w2x2, ids, w)
    assert np.array_equal(bf16_f64(y2), 2.0 * bf16_f64(y1))


def test_zero_inputs_give_zero():
    p, x, w13, w2, ids, w = small_problem(M=4, seed=8)
    y = oracle.fused_experts_bf16(np.zeros_like(x), w13, w2, ids, w)
    assert np.all(bf16_f64(y) == 0.0)
    w13z = w13.copy()
    w13z[:, p.I:, :] = 0                                           # up half zero
    y = oracle.fused_experts_bf16(x, w13z, w2, ids, w)
    assert np.all(bf16_f64(y) == 0.0)


def test_slot_order_and_weights_enter_the_sum():
    # swapping two slots (ids and weights together) leaves y unchanged; swapping
    # only the weights changes it
    _, x, w13, w2, ids, w = small_problem(M=5, E=4, k=2, seed=9)
    y = oracle.fused_experts_bf16(x, w13, w2, ids, w)
    y_sw = oracle.fused_experts_bf16(x, w13, w2, ids[:, ::-1].copy(), w[:, ::-1].copy())
    assert np.all(np.abs(bf16_f64(y) - bf16_f64(y_sw)) <= 2.0 ** -8 * np.abs(bf16_f64(y)))
    y_bad = oracle.fused_experts_bf16(x, w13, w2, ids, w[:, ::-1].copy())
    assert not np.allclose(bf16_f64(y), bf16_f64(y_bad), rtol=1e-2)


# ------------------------------------------------------------------ fp8 ---

def lossless_fp8(shape_blocks, rng):
    """A [N, K] matrix of e4m3 codes with one power-of-two scale per 128x128
    block and a 448 code in every block, so that re-quantising it is exact."""
    nb, kb = shape_blocks
    codes = rng.integers(0, 0x7E, (nb * 128, kb * 128)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape).astype(np.uint8) << 7)
    codes[::128, ::128] = 0x7E                                     # amax code in each block
    exps = rng.integers(-9, -3, (nb, kb))
    scale = (2.0 ** exps).astype(np.float32)
    return codes, scale


def test_fp8_gemm_lossless_equals_bf16_gemm():
    rng = np.random.default_rng(12)
    N, K = 384, 512
    qw, sw = lossless_fp8((N // 128, K // 128), rng)
    wreal = e4m3_f64(qw) * np.repeat(np.repeat(sw, 128, 0), 128, 1)
    wb = bits16(torch.from_numpy(wreal).to(torch.bfloat16))        # exact: 4 significant bits
    assert np.array_equal(bf16_f64(wb), wreal)
    # activation row: one power-of-two scale per 128 group
    qa = rng.integers(0, 0x7E, K).astype(np.uint8)
    qa[::128] = 0x7E
    sa = (2.0 ** rng.integers(-4, 3, K // 128)).astype(np.float32)
    areal = e4m3_f64(qa) * np.repeat(sa, 128)
    ab = bits16(torch.from_numpy(areal).to(torch.bfloat16))
    # quantising the real activation row gives back the same codes and scales
    q2, s2 = oracle.quant_groups_fp8(areal[None, :].astype(np.float32))
    assert np.array_equal(q2[0], qa) and np.array_equal(s2[0], sa)
    h8 = oracle.gemm_fp8(qa, sa, qw, sw)
    hb = oracle.gemm1_bf16(ab, wb)         # gemm1 treats K=H and N=2I
    assert np.array_equal(h8, hb)
    # transposing the weight-scale grid must break it (it is not symmetric)
    h8t = oracle.gemm_fp8(qa, sa, qw, np.ascontiguousarray(sw.T).reshape(sw.shape))
    assert not np.array_equal(h8t, hb)


def test_fp8_gemm_against_numpy_general():
    rng = np.random.default_rng(13)
    N, K = 256, 384
    w = torch.from_numpy(rng.standard_normal((N, K)) / np.sqrt(K)).to(torch.bfloat16)
    qw_t, sw_t = synth.block_quant_fp8(w)
    qw, sw = bits8(qw_t), sw_t.numpy()
    a = rng.standard_normal((1, K)).astype(np.float32)
    qa, sa = oracle.quant_groups_fp8(a)
    out = oracle.gemm_fp8(qa[0], sa[0], qw, sw)
    wreal = e4m3_f64(qw) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    areal = e4m3_f64(qa[0]) * np.repeat(sa[0].astype(np.float64), 128)
    ref = wreal @ areal
    assert np.all(np.abs(bf16_f64(out) - ref) <= RNE * np.abs(ref) + 1e-12)


def test_fp8_act_quantises_silu_mul():
    rng = np.random.default_rng(14)
    I = 256
    h = bits16(torch.from_numpy(rng.standard_normal(2 * I) * 2).to(torch.bfloat16))
    hf = bf16_f64(h)
    for alpha in (1.0, 0.37):
        zq, zs = oracle.act_fp8(h, alpha)
        zf = alpha * silu(hf[:I]) * hf[I:]
        amax = np.abs(zf).reshape(-1, 128).max(1)
        np.testing.assert_allclose(zs, amax / 448.0, rtol=2e-7)
        deq = e4m3_f64(zq) * np.repeat(zs.astype(np.float64), 128)
        s = np.repeat(zs.astype(np.float64), 128)
        assert np.all(np.abs(deq - zf) <= 2.0 ** -4 * np.abs(zf) + 2.0 ** -10 * s + 1e-12)


def test_fp8_layer_close_to_bf16_layer_on_same_weights():
    p = synth.Problem(M=6, H=256, I=256, E=3, topk=2, wdtype="fp8", seed=3)
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), 2)
    x = bits16(inp.x)
    y8 = oracle.fused_experts_fp8(x, bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q),
                                  inp.w2s.numpy(), ids, w)
    # the bf16 layer on the dequantised weights
    d13 = inp.w13q.double() * inp.w13s.double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    d2 = inp.w2q.double() * inp.w2s.double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    yb = oracle.fused_experts_bf16(x, bits16(d13.to(torch.bfloat16)), bits16(d2.to(torch.bfloat16)),
                                   ids, w)
    a, b = bf16_f64(y8), bf16_f64(yb)
    # x and z carry e4m3's 3-bit mantissa (<= 2^-4 relative per value), so the
    # agreement is statistical: about 4-5 % relative RMS on these shapes
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 0.005 < rel < 0.08, rel


def test_fp8_on_input_equals_on_output_for_power_of_two_weights():
    p = synth.Problem(M=4, H=256, I=256, E=3, topk=2, wdtype="fp8", seed=4)
    inp = synth.make_inputs(p, "cpu")
    ids, _ = oracle.topk(inp.logits.numpy(), 2)
    w = np.tile(np.array([0.5, 0.25], np.float32), (4, 1))
    args = (bits16(inp.x), bits8(inp.w13q), inp.w13s.numpy(), bits8(inp.w2q), inp.w2s.numpy(),
            ids, w)
    # z is quantised with a per-group scale, which absorbs a power-of-two factor
    assert np.array_equal(oracle.fused_experts_fp8(*args, on_input=True),
                          oracle.fused_experts_fp8(*args, on_input=False))


@pytest.mark.parametrize("name", ["tiny"])
def test_named_workload_oracle_runs(name):
    p = synth.Problem.named(name)
    inp = synth.make_inputs(p, "cpu")
    ids, w = oracle.topk(inp.logits.numpy(), p.topk)
    y = oracle.fused_experts_bf16(bits16(inp.x), bits16(inp.w13), bits16(inp.w2), ids, w)
    assert y.shape == (p.M, p.H) and np.all(np.isfinite(bf16_f64(y)))
