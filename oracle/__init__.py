"""CPU oracle for the fused MoE expert forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never loads it, and it
never loads the HIP library. The arithmetic lives in ``moe_oracle.c`` (plain
per-token loops, fp64 accumulation, bf16 rounding at h, z, o and y); this file
only marshals numpy arrays.

Functions with no independent pin would say "parity unpinned" here; every
function below is pinned by the CPU tests (``tests/test_oracle_*.py``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_SO names another build of the same source (the sanitizer build of
# tests/test_oracle_sanitized.py); by default the in-tree library
_SO = os.environ.get("MOE_ORACLE_SO") or os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        sig = {
            "oracle_bf16_to_f64_n": [_P, _I64, _P],
            "oracle_f64_to_bf16_n": [_P, _I64, _P],
            "oracle_e4m3_to_f64_n": [_P, _I64, _P],
            "oracle_f32_to_e4m3_n": [_P, _I64, _P],
            "oracle_quant_groups_fp8": [_P, _I64, _P, _P],
            "oracle_topk": [_P, _I64, _I32, _I32, _I32, _P, _P],
            "oracle_e8m0_to_f64": [ctypes.c_uint8],
            "oracle_e2m1_to_f64": [ctypes.c_uint8],
            "oracle_f32_to_e2m1": [ctypes.c_float],
            "oracle_quant_mx_fp8": [_P, _I64, _P, _P],
            "oracle_quant_mx_fp4": [_P, _I64, _P, _P],
            "oracle_gemm_mx": [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _P],
            "oracle_fused_experts_mx": [_I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                        _I32, _I64, _I64, _P, _P],
            "oracle_topk_grouped": [_P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                                    ctypes.c_float, _P, _P],
            "oracle_align_capacity": [_I64, _I32, _I32, _I32],
            "oracle_align": [_P, _I64, _I32, _I32, _I32, _I64, _P, _I32, _P, _P, _P, _P],
            "oracle_gemm1_bf16": [_P, _P, _I32, _I32, _P],
            "oracle_act_bf16": [_P, _I32, ctypes.c_double, _P],
            "oracle_gemm2_bf16": [_P, _P, _I32, _I32, _P],
            "oracle_gemm_fp8": [_P, _P, _P, _P, _I32, _I32, _P],
            "oracle_act_fp8": [_P, _I32, ctypes.c_double, _P, _P],
            "oracle_fused_experts_bf16": [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                          _I32, _P, _I32, _I64, _I64, _P, _P],
            "oracle_fused_experts_fp8": [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                         _P, _P, _I32, _P, _I32, _I64, _I64, _P, _P],
            "oracle_dense_experts_bf16": [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                          _P, _P],
            "oracle_batched_experts_bf16": [_I32, _I64, _I32, _I32, _P, _P, _P, _P, _P],
            "oracle_batched_experts_fp8": [_I32, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
        L.oracle_align_capacity.restype = _I64
        L.oracle_e8m0_to_f64.restype = ctypes.c_double
        L.oracle_e2m1_to_f64.restype = ctypes.c_double
        L.oracle_f32_to_e2m1.restype = ctypes.c_uint8
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = _I32
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_threads())


# ---------------------------------------------------------------- codecs ---

def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().oracle_bf16_to_f64_n(_p(b), b.size, _p(out))
    return out


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    v = _c(np.asarray(v, np.float64), np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_bf16_n(_p(v), v.size, _p(out))
    return out


def e4m3_to_f64(c: np.ndarray) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_to_f64_n(_p(c), c.size, _p(out))
    return out


def f32_to_e4m3(v: np.ndarray) -> np.ndarray:
    v = _c(np.asarray(v, np.float32), np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_f32_to_e4m3_n(_p(v), v.size, _p(out))
    return out


def quant_groups_fp8(v: np.ndarray):
    """Per-row, per-128-column dynamic fp8 quantisation of a [rows, n] fp32 array."""
    v = _c(np.asarray(v, np.float32), np.float32)
    rows, n = v.shape
    assert n % 128 == 0
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, n // 128), np.float32)
    for r in range(rows):
        lib().oracle_quant_groups_fp8(_p(v[r]), n, _p(q[r]), _p(s[r]))
    return q, s


# ---------------------------------------------------------------- router ---

def topk(logits: np.ndarray, k: int, renormalize: bool = True):
    logits = _c(logits, np.float32)
    M, E = logits.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float32)
    rc = lib().oracle_topk(_p(logits), M, E, k, int(renormalize), _p(ids), _p(w))
    if rc:
        raise ValueError("oracle_topk: invalid arguments")
    return ids, w


def topk_grouped(logits: np.ndarray, k: int, scoring: str = "softmax", renormalize: bool = True,
                 num_expert_group: int = 1, topk_group: int = 1, bias: np.ndarray | None = None,
                 routed_scaling_factor: float = 1.0):
    """Grouped / sigmoid router -> (ids int32 [M, k], weights fp32 [M, k])."""
    logits = _c(logits, np.float32)
    M, E = logits.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float32)
    b = None if bias is None else _c(bias, np.float32)
    rc = lib().oracle_topk_grouped(_p(logits), M, E, k, {"softmax": 0, "sigmoid": 1}[scoring],
                                   int(renormalize), num_expert_group, topk_group,
                                   _p(b) if b is not None else None, float(routed_scaling_factor),
                                   _p(ids), _p(w))
    if rc:
        raise ValueError("oracle_topk_grouped: invalid arguments")
    return ids, w


# ----------------------------------------------------------------- align ---

def align_capacity(M: int, k: int, E: int, B: int) -> int:
    return int(lib().oracle_align_capacity(M, k, E, B))


def _emap(expert_map):
    """(pointer-ready map, its length) or (None, 0): ids are local without a map."""
    if expert_map is None:
        return None, 0
    m = _c(expert_map, np.int32)
    return m, int(m.size)


def align(ids: np.ndarray, E: int, B: int, cap: int | None = None, expert_map=None):
    """With expert_map (global id -> local expert or -1), E is the local expert
    count and items of remote experts get no row (inv_perm -1)."""
    ids = _c(ids, np.int32)
    M, k = ids.shape
    if cap is None:
        cap = align_capacity(M, k, E, B)
    emap, eg = _emap(expert_map)
    sorted_ids = np.empty(cap, np.int32)
    expert_ids = np.empty(cap // B, np.int32)
    npp = np.zeros(1, np.int32)
    inv = np.empty((M, k), np.int32)
    rc = lib().oracle_align(_p(ids), M, k, E, B, cap, _p(emap) if emap is not None else None, eg,
                            _p(sorted_ids), _p(expert_ids), _p(npp), _p(inv))
    if rc:
        raise ValueError(f"oracle_align failed ({rc})")
    return sorted_ids, expert_ids, int(npp[0]), inv


# ------------------------------------------------------------ expert steps ---

def gemm1_bf16(x_row: np.ndarray, w13e: np.ndarray) -> np.ndarray:
    x_row = _c(x_row, np.uint16)
    w13e = _c(w13e, np.uint16)
    N2, H = w13e.shape
    h = np.empty(N2, np.uint16)
    lib().oracle_gemm1_bf16(_p(x_row), _p(w13e), H, N2 // 2, _p(h))
    return h


def act_bf16(h: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    h = _c(h, np.uint16)
    I = h.size // 2
    z = np.empty(I, np.uint16)
    lib().oracle_act_bf16(_p(h), I, float(alpha), _p(z))
    return z


def gemm2_bf16(z: np.ndarray, w2e: np.ndarray) -> np.ndarray:
    z = _c(z, np.uint16)
    w2e = _c(w2e, np.uint16)
    H, I = w2e.shape
    o = np.empty(H, np.uint16)
    lib().oracle_gemm2_bf16(_p(z), _p(w2e), H, I, _p(o))
    return o


def gemm_fp8(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    qa, sa = _c(qa, np.uint8), _c(sa, np.float32)
    qw, sw = _c(qw, np.uint8), _c(sw, np.float32)
    N, K = qw.shape
    out = np.empty(N, np.uint16)
    lib().oracle_gemm_fp8(_p(qa), _p(sa), _p(qw), _p(sw), N, K, _p(out))
    return out


def act_fp8(h: np.ndarray, alpha: float = 1.0):
    h = _c(h, np.uint16)
    I = h.size // 2
    zq = np.empty(I, np.uint8)
    zs = np.empty(I // 128, np.float32)
    lib().oracle_act_fp8(_p(h), I, float(alpha), _p(zq), _p(zs))
    return zq, zs


# ----------------------------------------------------------------- layer ---

def fused_experts_bf16(x, w13, w2, ids, weights, on_input=False, t0=0, t1=None,
                       return_acc=False, expert_map=None):
    """y rows [t0, t1) of the layer with bf16 weights (uint16 bit patterns).
    With expert_map, w13/w2 hold the local experts and ids are global."""
    x, w13, w2 = _c(x, np.uint16), _c(w13, np.uint16), _c(w2, np.uint16)
    ids, weights = _c(ids, np.int32), _c(weights, np.float32)
    M, H = x.shape
    E, N2, _ = w13.shape
    k = ids.shape[1]
    t1 = M if t1 is None else t1
    y = np.zeros((M, H), np.uint16)
    acc = np.zeros((M, H), np.float64) if return_acc else None
    emap, eg = _emap(expert_map)
    rc = lib().oracle_fused_experts_bf16(M, H, N2 // 2, E, k, _p(x), _p(w13), _p(w2), _p(ids),
                                         _p(weights), int(on_input),
                                         _p(emap) if emap is not None else None, eg, t0, t1,
                                         _p(y), _p(acc) if acc is not None else None)
    if rc:
        raise ValueError("oracle_fused_experts_bf16: expert id out of range")
    return (y[t0:t1], acc[t0:t1]) if return_acc else y[t0:t1]


def fused_experts_fp8(x, w13q, w13s, w2q, w2s, ids, weights, on_input=False, t0=0, t1=None,
                      return_acc=False, expert_map=None):
    """y rows [t0, t1) of the layer with e4m3 weights and 128x128 block scales."""
    x = _c(x, np.uint16)
    w13q, w2q = _c(w13q, np.uint8), _c(w2q, np.uint8)
    w13s, w2s = _c(w13s, np.float32), _c(w2s, np.float32)
    ids, weights = _c(ids, np.int32), _c(weights, np.float32)
    M, H = x.shape
    E, N2, _ = w13q.shape
    k = ids.shape[1]
    t1 = M if t1 is None else t1
    y = np.zeros((M, H), np.uint16)
    acc = np.zeros((M, H), np.float64) if return_acc else None
    emap, eg = _emap(expert_map)
    rc = lib().oracle_fused_experts_fp8(M, H, N2 // 2, E, k, _p(x), _p(w13q), _p(w13s),
                                        _p(w2q), _p(w2s), _p(ids), _p(weights), int(on_input),
                                        _p(emap) if emap is not None else None, eg,
                                        t0, t1, _p(y), _p(acc) if acc is not None else None)
    if rc:
        raise ValueError("oracle_fused_experts_fp8: expert id out of range")
    return (y[t0:t1], acc[t0:t1]) if return_acc else y[t0:t1]


def dense_experts_bf16(x, w13, w2, ids, weights, return_acc=False):
    """Every expert evaluated for every token, weighted 0 outside the top-k."""
    x, w13, w2 = _c(x, np.uint16), _c(w13, np.uint16), _c(w2, np.uint16)
    ids, weights = _c(ids, np.int32), _c(weights, np.float32)
    M, H = x.shape
    E, N2, _ = w13.shape
    k = ids.shape[1]
    y = np.zeros((M, H), np.uint16)
    acc = np.zeros((M, H), np.float64)
    lib().oracle_dense_experts_bf16(M, H, N2 // 2, E, k, _p(x), _p(w13), _p(w2), _p(ids),
                                    _p(weights), _p(y), _p(acc))
    return (y, acc) if return_acc else y


# ---------------------------------------------------------- batched form ---

def batched_experts_bf16(a, counts, w13, w2):
    """out [E, max_M, H] (uint16 bf16 bits): expert e applied, unweighted, to rows
    i < counts[e] of its batch a[e]; other rows 0."""
    a, w13, w2 = _c(a, np.uint16), _c(w13, np.uint16), _c(w2, np.uint16)
    counts = _c(counts, np.int32)
    E, max_M, H = a.shape
    I = w13.shape[1] // 2
    out = np.empty((E, max_M, H), np.uint16)
    if lib().oracle_batched_experts_bf16(E, max_M, H, I, _p(a), _p(counts), _p(w13), _p(w2), _p(out)):
        raise ValueError("oracle_batched_experts_bf16: negative count")
    return out


def batched_experts_fp8(a, counts, w13q, w13s, w2q, w2s):
    """The batched form with e4m3 weights and 128x128 block scales."""
    a, counts = _c(a, np.uint16), _c(counts, np.int32)
    w13q, w2q = _c(w13q, np.uint8), _c(w2q, np.uint8)
    w13s, w2s = _c(w13s, np.float32), _c(w2s, np.float32)
    E, max_M, H = a.shape
    I = w13q.shape[1] // 2
    out = np.empty((E, max_M, H), np.uint16)
    if lib().oracle_batched_experts_fp8(E, max_M, H, I, _p(a), _p(counts), _p(w13q), _p(w13s),
                                        _p(w2q), _p(w2s), _p(out)):
        raise ValueError("oracle_batched_experts_fp8: negative count")
    return out


# ------------------------------------------------------------- MX formats ---

def e8m0_to_f64(c: int) -> float:
    return float(lib().oracle_e8m0_to_f64(int(c)))


def e2m1_to_f64(c: int) -> float:
    return float(lib().oracle_e2m1_to_f64(int(c)))


def f32_to_e2m1(v: float) -> int:
    return int(lib().oracle_f32_to_e2m1(float(v)))


def quant_mx_fp8(v: np.ndarray):
    """[.., K] values -> (E4M3 codes [.., K] uint8, E8M0 codes [.., K/32] uint8), per 32 columns."""
    v = _c(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    sc = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    lib().oracle_quant_mx_fp8(_p(v), v.size, _p(q), _p(sc))
    return q, sc


def quant_mx_fp4(v: np.ndarray):
    """[.., K] values -> (E2M1 codes [.., K/2] uint8, two per byte, element 2i low, E8M0 [.., K/32])."""
    v = _c(v, np.float32)
    q = np.empty(v.shape[:-1] + (v.shape[-1] // 2,), np.uint8)
    sc = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    lib().oracle_quant_mx_fp4(_p(v), v.size, _p(q), _p(sc))
    return q, sc


def gemm_mx(qa, sa, qw, sw, fmt_w="e4m3"):
    """bf16 [N] = MX GEMM of one activation row (E4M3 + E8M0 [K/32] or fp32 [K/128]) with
    weights (E4M3 [N, K] or E2M1 [N, K/2]) and their E8M0 scales [N, K/32]."""
    qa, qw, sw = _c(qa, np.uint8), _c(qw, np.uint8), _c(sw, np.uint8)
    mx_a = sa.dtype == np.uint8
    sa = _c(sa, np.uint8 if mx_a else np.float32)
    N, K = sw.shape[0], sw.shape[1] * 32
    out = np.empty(N, np.uint16)
    lib().oracle_gemm_mx(_p(qa), _p(sa), int(mx_a), _p(qw), _p(sw), 0 if fmt_w == "e4m3" else 1, N, K, _p(out))
    return out


def fused_experts_mx(x, w13q, w13e, w2q, w2e, ids, weights, w4=False, on_input=False, t0=0, t1=None,
                     return_acc=False):
    """y rows [t0, t1): MXFP8 layer (w4=False: E4M3 weights, MXFP8 activations and z) or
    W4A8 (w4=True: E2M1 weights [E, N, K/2], FP8 activations and z with fp32 per-128 scales);
    weight scales E8M0 [E, N, K/32] in both."""
    x = _c(x, np.uint16)
    w13q, w13e, w2q, w2e = (_c(a, np.uint8) for a in (w13q, w13e, w2q, w2e))
    ids, weights = _c(ids, np.int32), _c(weights, np.float32)
    M, H = x.shape
    E, N2 = w13e.shape[0], w13e.shape[1]
    k = ids.shape[1]
    t1 = M if t1 is None else t1
    y = np.zeros((M, H), np.uint16)
    acc = np.zeros((M, H), np.float64) if return_acc else None
    rc = lib().oracle_fused_experts_mx(M, H, N2 // 2, E, k, int(w4), _p(x), _p(w13q), _p(w13e), _p(w2q),
                                       _p(w2e), _p(ids), _p(weights), int(on_input), t0, t1, _p(y),
                                       _p(acc) if acc is not None else None)
    if rc:
        raise ValueError("oracle_fused_experts_mx: expert id out of range")
    return (y[t0:t1], acc[t0:t1]) if return_acc else y[t0:t1]
