"""The C ABI library on the CPU: it loads, exports every declared symbol, and
every host-side check returns its status before any launch."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import mixture_experts_ffn_block_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = "\n".join(l for l in src.splitlines() if not l.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    for n in names:
        assert getattr(L, n) is not None


def test_library_exports_nothing_else():
    # internal launchers and helpers have hidden visibility
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    funcs = {l.split()[-1] for l in out.splitlines() if len(l.split()) == 3 and l.split()[1] == "T"}
    assert funcs == set(declared_functions()), sorted(funcs ^ set(declared_functions()))


def test_capacity_matches_oracle():
    for args in [(64, 2, 8, 16), (4096, 2, 8, 128), (8192, 8, 256, 128), (32, 8, 128, 16),
                 (1, 1, 1, 16), (0, 2, 8, 16), (7, 3, 5, 64)]:
        assert moe.moe_align_capacity(*args) == oracle.align_capacity(*args)
    assert moe.moe_align_capacity(-1, 2, 8, 16) == -1


def P(**kw):
    d = dict(M=64, H=256, I=512, E=8, topk=2, block_m=16, wdtype=moe.MOE_W_BF16, on_input=False)
    d.update(kw)
    return moe.make_problem(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), moe.MOE_E_INVALID),
    (dict(topk=0), moe.MOE_E_INVALID),
    (dict(topk=9), moe.MOE_E_INVALID),
    (dict(E=300, topk=2), moe.MOE_E_UNSUPPORTED),
    (dict(H=200), moe.MOE_E_UNSUPPORTED),
    (dict(I=96), moe.MOE_E_UNSUPPORTED),
    (dict(block_m=48), moe.MOE_E_UNSUPPORTED),
    (dict(wdtype=7), moe.MOE_E_UNSUPPORTED),
    (dict(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=16), moe.MOE_E_UNSUPPORTED),
    (dict(weight_layout=2), moe.MOE_E_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_TILED, block_m=64), moe.MOE_E_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_TILED, block_m=32), moe.MOE_E_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_TILED, block_m=128, wdtype=moe.MOE_W_FP8_E4M3_BLOCK128),
     moe.MOE_E_UNSUPPORTED),
    # row blocks x column tiles of the GEMM grids past int32 (2^26 tokens, top-8, block_m 16)
    (dict(M=1 << 26, topk=8, E=256, H=4096, I=14336), moe.MOE_E_UNSUPPORTED),
])
def test_fused_experts_validation(kw, status):
    p = P(**kw)
    assert moe.moe_workspace_bytes(p) == 0
    dummy = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = moe.lib().fused_experts(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                 dummy, dummy, 1 << 40, None)
    assert rc == status


def test_large_problem_below_the_grid_limit_is_accepted():
    # 2^20 tokens of the same shape: 64 Ki row blocks x 225 column tiles fit
    assert moe.moe_workspace_bytes(P(M=1 << 20, topk=8, E=256, H=4096, I=14336)) > 0


def test_fused_experts_pointer_and_workspace_checks():
    p = P()
    need = moe.moe_workspace_bytes(p)
    assert need > 0
    d = ctypes.c_void_p(1 << 20)
    L = moe.lib()
    assert L.fused_experts(ctypes.byref(p), None, d, None, d, None, d, d, d, d, need, None) \
        == moe.MOE_E_INVALID
    assert L.fused_experts(ctypes.byref(p), d, d, None, d, None, d, d, d, d, need - 1, None) \
        == moe.MOE_E_WORKSPACE
    assert L.fused_experts(ctypes.byref(p), d, d, None, d, None, d, d, d, None, need, None) \
        == moe.MOE_E_WORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 64)
    assert L.fused_experts(ctypes.byref(p), d, d, None, d, None, d, d, d, misaligned, need, None) \
        == moe.MOE_E_INVALID
    pf = P(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=64)
    needf = moe.moe_workspace_bytes(pf)
    assert L.fused_experts(ctypes.byref(pf), d, d, None, d, d, d, d, d, d, needf, None) \
        == moe.MOE_E_INVALID
    assert L.fused_experts(ctypes.byref(P(M=0)), None, None, None, None, None, None, None, None,
                           None, 0, None) == moe.MOE_OK


def test_workspace_grows_with_problem():
    a = moe.moe_workspace_bytes(P(M=64))
    b = moe.moe_workspace_bytes(P(M=128))
    c = moe.moe_workspace_bytes(P(M=64, wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=32))
    assert 0 < a < b and c > 0 and a % 256 == 0


def test_router_align_quant_validation():
    L = moe.lib()
    d = ctypes.c_void_p(1 << 20)
    assert L.moe_topk(d, 4, 8, 9, 1, d, d, None) == moe.MOE_E_INVALID
    assert L.moe_topk(d, 4, 300, 2, 1, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_topk(None, 4, 8, 2, 1, d, d, None) == moe.MOE_E_INVALID
    assert L.moe_topk(None, 0, 8, 2, 1, None, None, None) == moe.MOE_OK
    assert L.moe_align_block_size(d, 4, 2, 8, 24, d, d, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_align_block_size(d, 4, 2, 8, 16, d, d, None, d, None) == moe.MOE_E_INVALID
    assert L.moe_align_block_size(None, 4, 2, 8, 16, d, d, d, d, None) == moe.MOE_E_INVALID
    assert L.moe_quant_fp8_groups(d, 4, 100, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_quant_fp8_groups(None, 4, 128, d, d, None) == moe.MOE_E_INVALID
    assert L.moe_quant_fp8_groups(None, 0, 128, None, None, None) == moe.MOE_OK
    for s in range(5):
        assert moe.status_string(s)


def test_pack_weights_validation():
    L = moe.lib()
    p = P(weight_layout=moe.MOE_LAYOUT_TILED)
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 40)
    assert L.moe_pack_weights(ctypes.byref(p), 3, a, b, None) == moe.MOE_E_INVALID
    assert L.moe_pack_weights(ctypes.byref(p), 1, None, b, None) == moe.MOE_E_INVALID
    assert L.moe_pack_weights(ctypes.byref(p), 2, a, None, None) == moe.MOE_E_INVALID
    # w13 of this problem is 8 * 1024 * 256 * 2 bytes: a destination inside it overlaps
    inside = ctypes.c_void_p((1 << 20) + 4096)
    assert L.moe_pack_weights(ctypes.byref(p), 1, a, inside, None) == moe.MOE_E_INVALID
    assert L.moe_pack_weights(ctypes.byref(p), 1, a, ctypes.c_void_p((1 << 40) + 8), None) \
        == moe.MOE_E_INVALID  # 16-byte alignment
    pf = P(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=128)
    assert L.moe_pack_weights(ctypes.byref(pf), 1, a, b, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_pack_weights(ctypes.byref(P(H=200)), 1, a, b, None) == moe.MOE_E_UNSUPPORTED


def test_problem_struct_matches_header():
    # the ctypes mirror of moe_problem_t has the header's fields in the header's order
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    body = re.search(r"typedef struct \{(.*?)\} moe_problem_t;", src, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int64_t|int32_t)\s+([^;]+);", body)
    names = [n.strip() for _, decl in fields for n in decl.split(",")]
    assert names == [f[0] for f in moe.MoeProblem._fields_]
    kinds = [k for k, decl in fields for _ in decl.split(",")]
    assert [ctypes.sizeof(f[1]) for f in moe.MoeProblem._fields_] == [8 if k == "int64_t" else 4 for k in kinds]


def test_expert_parallel_validation():
    L = moe.lib()
    d = ctypes.c_void_p(1 << 20)
    # an expert-parallel problem: 256 global experts, 4 held here, top-8 over the global range
    p = P(M=64, E=4, topk=8, num_global_experts=256, block_m=128)
    need = moe.moe_workspace_bytes(p)
    assert need > 0
    assert L.fused_experts(ctypes.byref(p), d, d, None, d, None, d, d, d, d, need, None) == moe.MOE_E_INVALID
    assert L.fused_experts_ep(ctypes.byref(p), None, d, d, None, d, None, d, d, d, d, need, None) \
        == moe.MOE_E_INVALID
    assert L.fused_experts_ep(ctypes.byref(p), d, d, d, None, d, None, d, d, d, d, need - 1, None) \
        == moe.MOE_E_WORKSPACE
    plain = P()
    assert L.fused_experts_ep(ctypes.byref(plain), d, d, d, None, d, None, d, d, d, d, 1 << 30, None) \
        == moe.MOE_E_INVALID                                       # no global range given
    assert moe.moe_workspace_bytes(P(E=4, topk=8)) == 0            # top-8 of 4 local experts
    assert moe.moe_workspace_bytes(P(num_global_experts=-1)) == 0
    assert moe.moe_workspace_bytes(P(num_global_experts=1 << 17)) == 0
    assert L.fused_experts_ep(ctypes.byref(P(M=0, E=4, topk=8, num_global_experts=256)), d, None, None,
                              None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    A = L.moe_align_block_size_ep
    assert A(d, 4, 8, 4, d, 4, 16, d, d, d, d, None) == moe.MOE_E_INVALID     # topk > global experts
    assert A(d, 4, 2, 256, None, 4, 16, d, d, d, d, None) == moe.MOE_E_INVALID
    assert A(d, 4, 2, 256, d, 300, 16, d, d, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert A(d, 4, 2, 256, d, 4, 24, d, d, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert A(None, 4, 2, 256, d, 4, 16, d, d, d, d, None) == moe.MOE_E_INVALID


def test_batched_validation():
    L = moe.lib()
    d = ctypes.c_void_p(1 << 20)
    p = P(M=32, E=8, topk=1)
    need = moe.moe_batched_workspace_bytes(p)
    assert need > 0
    for bad in (P(M=32, E=8, topk=2), P(M=32, E=8, topk=1, on_input=True),
                P(M=32, E=8, topk=1, num_global_experts=16)):
        assert moe.moe_batched_workspace_bytes(bad) == 0
        assert L.moe_batched_experts(ctypes.byref(bad), d, d, d, None, d, None, d, d, need, None) \
            == moe.MOE_E_INVALID
    assert L.moe_batched_experts(ctypes.byref(p), d, None, d, None, d, None, d, d, need, None) \
        == moe.MOE_E_INVALID
    assert L.moe_batched_experts(ctypes.byref(p), d, d, d, None, d, None, d, d, need - 1, None) \
        == moe.MOE_E_WORKSPACE
    assert L.moe_batched_experts(ctypes.byref(P(M=32, E=8, topk=1, block_m=48)), d, d, d, None, d, None,
                                 d, d, need, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_batched_experts(ctypes.byref(P(M=0, E=8, topk=1)), None, None, None, None, None, None,
                                 None, None, 0, None) == moe.MOE_OK


def test_grouped_router_validation():
    L = moe.lib()
    d = ctypes.c_void_p(1 << 20)
    T = L.moe_topk_grouped
    S, G = moe.MOE_SCORING_SOFTMAX, moe.MOE_SCORING_SIGMOID
    assert T(d, 4, 256, 8, 2, 1, 8, 4, None, 1.0, d, d, None) == moe.MOE_E_INVALID   # unknown scoring
    assert T(d, 4, 256, 8, S, 1, 7, 4, None, 1.0, d, d, None) == moe.MOE_E_INVALID   # 256 % 7
    assert T(d, 4, 256, 8, S, 1, 8, 9, None, 1.0, d, d, None) == moe.MOE_E_INVALID   # topk_group > G
    assert T(d, 4, 256, 40, S, 1, 8, 1, None, 1.0, d, d, None) == moe.MOE_E_INVALID  # 40 > 32
    assert T(d, 4, 64, 9, S, 1, 8, 1, None, 1.0, d, d, None) == moe.MOE_E_INVALID   # 9 > 1 * 8
    assert T(d, 4, 256, 8, S, 1, 8, 4, d, 1.0, d, d, None) == moe.MOE_E_INVALID     # bias with softmax
    assert T(d, 4, 64, 8, G, 1, 64, 64, d, 1.0, d, d, None) == moe.MOE_E_INVALID    # groups of one + bias
    assert T(d, 4, 384, 8, G, 1, 8, 4, d, 1.0, d, d, None) == moe.MOE_E_UNSUPPORTED
    assert T(d, 4, 256, 8, G, 1, 128, 64, None, 1.0, d, d, None) == moe.MOE_E_UNSUPPORTED  # G > 64
    assert T(None, 4, 256, 8, G, 1, 8, 4, d, 2.5, d, d, None) == moe.MOE_E_INVALID
    assert T(None, 0, 256, 8, G, 1, 8, 4, None, 2.5, None, None, None) == moe.MOE_OK


def test_chunked_workspace():
    full = moe.moe_workspace_bytes(P(M=1000, block_m=64))
    chunked = moe.moe_workspace_bytes(P(M=1000, block_m=64, chunk_tokens=256))
    assert chunked == moe.moe_workspace_bytes(P(M=256, block_m=64)) and chunked < full
    assert moe.moe_workspace_bytes(P(M=100, block_m=64, chunk_tokens=256)) == moe.moe_workspace_bytes(P(M=100, block_m=64))
    assert moe.moe_workspace_bytes(P(chunk_tokens=-1)) == 0


def test_weight_scale_shapes_are_checked_exactly():
    # the binding refuses scale tensors the kernels would read past (one expert's, a
    # rank's slice, a transposed grid, unpacked MX bytes) before anything is launched
    import torch
    E, H, I = 4, 512, 256
    f = lambda *s: torch.empty(s, dtype=torch.float32)
    w = lambda *s: torch.empty(s, dtype=torch.int32)
    fp8, mx, w4 = moe.MOE_W_FP8_E4M3_BLOCK128, moe.MOE_W_MXFP8, moe.MOE_W_W4A8_MXFP4
    moe.check_weight_scales(fp8, E, H, I, f(E, 4, 4), f(E, 4, 2), "t")
    moe.check_weight_scales(mx, E, H, I, w(E, 4, 512), w(E, 2, 512), "t")
    moe.check_weight_scales(w4, E, H, I, w(E, 4, 512), w(E, 2, 512), "t")
    moe.check_weight_scales(moe.MOE_W_BF16, E, H, I, None, None, "t")
    bad = [
        (fp8, f(1, 4, 4), f(E, 4, 2)),            # one expert's scales
        (fp8, f(E, 4, 4), f(E, 2, 4)),            # w2 grid transposed
        (fp8, f(E // 2, 4, 4), f(E // 2, 4, 2)),  # half of the experts
        (fp8, None, f(E, 4, 2)),
        (mx, w(E, 4, 512), w(E, 512, 2)),          # not the packed MN-major words
        (mx, w(E, 1024, 16), w(E, 2, 512)),        # unpacked [E, N, K/32] shape
        (w4, w(E, 4, 256), w(E, 2, 512)),
    ]
    for wd, a, b in bad:
        with pytest.raises(ValueError):
            moe.check_weight_scales(wd, E, H, I, a, b, "t")


def test_static_scratch_entry_point_validation():
    # fused_experts_static: the checks of fused_experts, an expert map refused, and a
    # problem whose scratch exceeds the library's 64 MiB array refused before any launch
    L = moe.lib()
    d = ctypes.c_void_p(1 << 20)
    for kw, status in [(dict(M=-1), moe.MOE_E_INVALID), (dict(topk=9), moe.MOE_E_INVALID),
                       (dict(H=200), moe.MOE_E_UNSUPPORTED), (dict(block_m=48), moe.MOE_E_UNSUPPORTED)]:
        assert L.fused_experts_static(ctypes.byref(P(**kw)), d, d, None, d, None, d, d, d, None) == status
    assert L.fused_experts_static(ctypes.byref(P(M=0)), None, None, None, None, None, None, None, None,
                                  None) == moe.MOE_OK
    assert L.fused_experts_static(ctypes.byref(P()), None, d, None, d, None, d, d, d, None) == moe.MOE_E_INVALID
    ep = moe.make_problem(64, 256, 512, 4, 2, 16, num_global_experts=8)
    assert L.fused_experts_static(ctypes.byref(ep), d, d, None, d, None, d, d, d, None) == moe.MOE_E_INVALID
    pf = P(wdtype=moe.MOE_W_FP8_E4M3_BLOCK128, block_m=64)
    assert L.fused_experts_static(ctypes.byref(pf), d, d, None, d, None, d, d, d, None) == moe.MOE_E_INVALID
    # the Mixtral-shaped prefill needs ~1.5 GB of scratch; the decode workload's fits
    big = moe.make_problem(4096, 4096, 14336, 8, 2, 256)
    assert L.fused_experts_static(ctypes.byref(big), d, d, None, d, None, d, d, d, None) == moe.MOE_E_WORKSPACE
    assert moe.moe_workspace_bytes(moe.make_problem(32, 2048, 768, 128, 8, 16)) < 64 << 20
