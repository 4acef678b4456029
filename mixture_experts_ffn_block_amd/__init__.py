"""Python binding of libmoe.so, the gfx950 fused MoE expert forward.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe.h``. torch supplies device memory
and the current HIP stream. If the library is not built this module raises
at import of the first call; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same sources (the host-sanitizer build of
# tests/test_sanitized.py); by default the in-tree library
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = range(5)
MOE_W_BF16, MOE_W_FP8_E4M3_BLOCK128, MOE_W_MXFP8, MOE_W_W4A8_MXFP4 = 0, 1, 2, 3
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = 0, 1
MOE_SCORING_SOFTMAX, MOE_SCORING_SIGMOID = 0, 1

EXPORTS = ("moe_topk", "moe_topk_grouped", "moe_align_capacity", "moe_align_block_size", "moe_align_block_size_ep",
           "moe_quant_fp8_groups", "moe_workspace_bytes", "fused_experts", "fused_experts_ep",
           "moe_expert_gemm_workspace_bytes",
           "moe_expert_gemm", "moe_silu_and_mul",
           "moe_expert_gemm_act_supported", "moe_expert_gemm_act", "moe_permute_scales",
           "moe_unpermute_reduce", "moe_pack_weights", "moe_batched_workspace_bytes",
           "moe_batched_experts", "moe_quant_mx_groups", "moe_pack_mx_scales", "moe_status_string",
           "fused_experts_static")


class MoeProblem(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("apply_router_weight_on_input", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("num_global_experts", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None
_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_topk.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P]
        L.moe_topk_grouped.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                                       ctypes.c_float, _P, _P, _P]
        L.moe_align_capacity.argtypes = [_I64, _I32, _I32, _I32]
        L.moe_align_capacity.restype = _I64
        L.moe_align_block_size.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P]
        L.moe_align_block_size_ep.argtypes = [_P, _I64, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P]
        L.moe_quant_fp8_groups.argtypes = [_P, _I64, _I32, _P, _P, _P]
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeProblem)]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.fused_experts.argtypes = [ctypes.POINTER(MoeProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]
        L.fused_experts_ep.argtypes = [ctypes.POINTER(MoeProblem), _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, ctypes.c_size_t, _P]
        L.fused_experts_static.argtypes = [ctypes.POINTER(MoeProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P]
        PP = ctypes.POINTER(MoeProblem)
        L.moe_expert_gemm_workspace_bytes.argtypes = [PP]
        L.moe_expert_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.moe_expert_gemm.argtypes = [PP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_silu_and_mul.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P]
        L.moe_permute_scales.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_expert_gemm_act_supported.argtypes = [PP]
        L.moe_expert_gemm_act_supported.restype = _I32
        L.moe_expert_gemm_act.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_unpermute_reduce.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_pack_weights.argtypes = [PP, _I32, _P, _P, _P]
        L.moe_quant_mx_groups.argtypes = [_P, _I64, _I32, _P, _P, _P]
        L.moe_pack_mx_scales.argtypes = [PP, _I32, _P, _P, _P]
        L.moe_batched_workspace_bytes.argtypes = [PP]
        L.moe_batched_workspace_bytes.restype = ctypes.c_size_t
        L.moe_batched_experts.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_status_string.argtypes = [_I32]
        L.moe_status_string.restype = ctypes.c_char_p
        for name in ("moe_topk", "moe_topk_grouped", "moe_align_block_size", "moe_align_block_size_ep",
                     "moe_quant_fp8_groups", "fused_experts", "fused_experts_ep",
                     "moe_expert_gemm", "moe_silu_and_mul", "moe_permute_scales",
                     "moe_expert_gemm_act", "moe_unpermute_reduce", "moe_pack_weights",
                     "moe_batched_experts", "moe_quant_mx_groups", "moe_pack_mx_scales",
                     "fused_experts_static"):
            getattr(L, name).restype = _I32
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().moe_status_string(s).decode()


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {dtype} device tensor, "
                         f"got {t.dtype} (contiguous={t.is_contiguous()}, device={t.device})")


def _need_size(t: torch.Tensor | None, dtypes, numel: int, name: str):
    """A device buffer the library will index up to `numel` elements of."""
    if t is None:
        raise ValueError(f"{name}: required")
    if t.dtype not in dtypes or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous device tensor of {dtypes}, got {t.dtype} "
                         f"(contiguous={t.is_contiguous()}, device={t.device})")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs {numel} elements, has {t.numel()}")


def weight_scale_shapes(wdtype: int, E: int, H: int, I: int):
    """Exact shapes of (w13_scale, w2_scale) for a weight format, or None for bf16: fp32
    128x128 blocks [E, 2I/128, H/128] and [E, H/128, I/128], or the packed E8M0 words of
    moe_pack_mx_scales [E, H/128, 2I] and [E, I/128, H] (MXFP8, W4A8)."""
    if wdtype == MOE_W_FP8_E4M3_BLOCK128:
        return (E, 2 * I // 128, H // 128), (E, H // 128, I // 128)
    if wdtype in (MOE_W_MXFP8, MOE_W_W4A8_MXFP4):
        return (E, H // 128, 2 * I), (E, I // 128, H)
    return None


def check_weight_scales(wdtype: int, E: int, H: int, I: int, w13_scale, w2_scale, what: str):
    """Raise ValueError unless both scale tensors have exactly the shapes the kernels index
    (a smaller tensor, e.g. one expert's or another rank's slice, would be read past its end)."""
    want = weight_scale_shapes(wdtype, E, H, I)
    if want is None:
        return
    for name, t, shape in (("w13_scale", w13_scale, want[0]), ("w2_scale", w2_scale, want[1])):
        if t is None:
            raise ValueError(f"{what}: {name} is required for this weight format")
        if tuple(t.shape) != shape:
            raise ValueError(f"{what}: {name} has shape {tuple(t.shape)}, expected {shape}")


_F8 = (torch.float8_e4m3fn, torch.uint8)
_BF = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_I32T = (torch.int32,)


# ----------------------------------------------------------------- entries ---

def moe_topk(logits: torch.Tensor, topk: int, renormalize: bool = True, stream=None,
             out: tuple[torch.Tensor, torch.Tensor] | None = None):
    """softmax + top-k router -> (topk_ids int32 [M, k], topk_weights fp32 [M, k])."""
    _need(logits, torch.float32, "logits")
    M, E = logits.shape
    if out is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
        w = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    else:
        ids, w = out
    _check(lib().moe_topk(_ptr(logits), M, E, topk, int(renormalize), _ptr(ids), _ptr(w),
                          _stream(stream)), "moe_topk")
    return ids, w


def moe_topk_grouped(logits: torch.Tensor, topk: int, scoring: str = "softmax", renormalize: bool = True,
                     num_expert_group: int = 1, topk_group: int = 1,
                     e_score_correction_bias: torch.Tensor | None = None,
                     routed_scaling_factor: float = 1.0, stream=None,
                     out: tuple[torch.Tensor, torch.Tensor] | None = None):
    """Grouped / sigmoid router -> (topk_ids int32 [M, k], topk_weights fp32 [M, k])."""
    _need(logits, torch.float32, "logits")
    if e_score_correction_bias is not None:
        _need(e_score_correction_bias, torch.float32, "e_score_correction_bias")
    M, E = logits.shape
    if out is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
        w = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    else:
        ids, w = out
    sc = {"softmax": MOE_SCORING_SOFTMAX, "sigmoid": MOE_SCORING_SIGMOID}[scoring]
    _check(lib().moe_topk_grouped(_ptr(logits), M, E, topk, sc, int(renormalize), num_expert_group,
                                  topk_group, _ptr(e_score_correction_bias), float(routed_scaling_factor),
                                  _ptr(ids), _ptr(w), _stream(stream)), "moe_topk_grouped")
    return ids, w


def moe_align_capacity(M: int, topk: int, E: int, block_m: int) -> int:
    return int(lib().moe_align_capacity(M, topk, E, block_m))


def moe_align_block_size(topk_ids: torch.Tensor, E: int, block_m: int, stream=None):
    """-> (sorted_token_ids [cap], expert_ids [cap/block_m], num_tokens_post_padded [1],
    inv_perm [M, topk]), all int32 on the device."""
    _need(topk_ids, torch.int32, "topk_ids")
    M, k = topk_ids.shape
    cap = moe_align_capacity(M, k, E, block_m)
    dev = topk_ids.device
    sorted_ids = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max(cap, 0) // block_m, dtype=torch.int32, device=dev)
    npp = torch.zeros(1, dtype=torch.int32, device=dev)
    inv = torch.empty((M, k), dtype=torch.int32, device=dev)
    _check(lib().moe_align_block_size(_ptr(topk_ids), M, k, E, block_m, _ptr(sorted_ids),
                                      _ptr(expert_ids), _ptr(npp), _ptr(inv), _stream(stream)),
           "moe_align_block_size")
    return sorted_ids, expert_ids, npp, inv


def moe_align_block_size_ep(topk_ids: torch.Tensor, expert_map: torch.Tensor, E: int, block_m: int,
                            stream=None):
    """Align on one expert-parallel rank: topk_ids are global, expert_map [G] int32 sends
    them to the E local experts or -1. Same outputs as moe_align_block_size."""
    _need(topk_ids, torch.int32, "topk_ids")
    _need(expert_map, torch.int32, "expert_map")
    M, k = topk_ids.shape
    cap = moe_align_capacity(M, k, E, block_m)
    dev = topk_ids.device
    sorted_ids = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max(cap, 0) // block_m, dtype=torch.int32, device=dev)
    npp = torch.zeros(1, dtype=torch.int32, device=dev)
    inv = torch.empty((M, k), dtype=torch.int32, device=dev)
    _check(lib().moe_align_block_size_ep(_ptr(topk_ids), M, k, expert_map.numel(), _ptr(expert_map),
                                         E, block_m, _ptr(sorted_ids), _ptr(expert_ids), _ptr(npp),
                                         _ptr(inv), _stream(stream)),
           "moe_align_block_size_ep")
    return sorted_ids, expert_ids, npp, inv


def moe_quant_fp8_groups(x: torch.Tensor, stream=None):
    """Per-row, per-128-column dynamic e4m3 quantisation -> (q, scale)."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    _check(lib().moe_quant_fp8_groups(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(stream)),
           "moe_quant_fp8_groups")
    return q, s


def make_problem(M, H, I, E, topk, block_m, wdtype=MOE_W_BF16, on_input=False,
                 weight_layout=MOE_LAYOUT_ROWS, num_global_experts=0, chunk_tokens=0) -> MoeProblem:
    return MoeProblem(M, H, I, E, topk, block_m, wdtype, int(on_input), weight_layout,
                      num_global_experts, chunk_tokens)


def moe_workspace_bytes(p: MoeProblem) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(p)))


def workspace_for(p: MoeProblem, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(p)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _layer_problem(x, w13, w2, topk_ids, topk_weights, block_m, w13_scale, w2_scale,
                   apply_router_weight_on_input, weight_layout, expert_map, chunk_tokens, what) -> MoeProblem:
    """Checks the layer's tensors (dtypes, contiguity, shapes, scale shapes) and returns the
    problem they describe."""
    if expert_map is not None:
        _need(expert_map, torch.int32, "expert_map")
    _need(x, torch.bfloat16, "x")
    w4 = w13.dtype == torch.uint8                  # E2M1 weights, two per byte (W4A8)
    fp8 = w13.dtype == torch.float8_e4m3fn or w4
    # e4m3 weights: fp32 128x128 block scales, or packed MX words (int32) from moe_pack_mx_scales
    mx = w13.dtype == torch.float8_e4m3fn and w13_scale is not None and w13_scale.dtype == torch.int32
    wdt = torch.uint8 if w4 else torch.float8_e4m3fn if fp8 else torch.bfloat16
    _need(w13, wdt, "w13")
    _need(w2, wdt, "w2")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_weights, torch.float32, "topk_weights")
    if fp8:
        _need(w13_scale, torch.int32 if (mx or w4) else torch.float32, "w13_scale")
        _need(w2_scale, torch.int32 if (mx or w4) else torch.float32, "w2_scale")
    M, H = x.shape
    E, N2, H2 = w13.shape
    d = 2 if w4 else 1
    if H2 * d != H or tuple(w2.shape) != (E, H, N2 // 2 // d) or topk_ids.shape != topk_weights.shape \
            or topk_ids.shape[0] != M:
        raise ValueError(f"{what}: inconsistent shapes")
    p = make_problem(M, H, N2 // 2, E, topk_ids.shape[1], block_m,
                     MOE_W_W4A8_MXFP4 if w4 else MOE_W_MXFP8 if mx else
                     MOE_W_FP8_E4M3_BLOCK128 if fp8 else MOE_W_BF16,
                     apply_router_weight_on_input, weight_layout,
                     0 if expert_map is None else expert_map.numel(), chunk_tokens)
    check_weight_scales(p.wdtype, E, H, N2 // 2, w13_scale, w2_scale, what)
    return p


def fused_experts(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, topk_ids: torch.Tensor,
                  topk_weights: torch.Tensor, block_m: int, w13_scale: torch.Tensor | None = None,
                  w2_scale: torch.Tensor | None = None, apply_router_weight_on_input=False,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None, weight_layout=MOE_LAYOUT_ROWS,
                  expert_map: torch.Tensor | None = None, chunk_tokens: int = 0) -> torch.Tensor:
    """y = fused MoE expert forward (bf16 [M, H]). `out` may be `x` (in place).

    weight_layout MOE_LAYOUT_TILED: w13 and w2 come from moe_pack_weights (same shapes).
    expert_map [G] int32 (one expert-parallel rank): topk_ids are global ids in [0, G),
    w13 / w2 hold this rank's E experts, and y sums only the slots of those experts.
    chunk_tokens > 0: the layer runs on chunks of that many tokens (workspace for one chunk)."""
    p = _layer_problem(x, w13, w2, topk_ids, topk_weights, block_m, w13_scale, w2_scale,
                       apply_router_weight_on_input, weight_layout, expert_map, chunk_tokens, "fused_experts")
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = workspace_for(p, x.device)
    if expert_map is None:
        _check(lib().fused_experts(ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                   _ptr(w2_scale), _ptr(topk_ids), _ptr(topk_weights), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(stream)),
               "fused_experts")
    else:
        _check(lib().fused_experts_ep(ctypes.byref(p), _ptr(expert_map), _ptr(x), _ptr(w13),
                                      _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(topk_ids),
                                      _ptr(topk_weights), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(stream)),
               "fused_experts_ep")
    return out


def fused_experts_static(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, topk_ids: torch.Tensor,
                         topk_weights: torch.Tensor, block_m: int, out: torch.Tensor,
                         w13_scale: torch.Tensor | None = None, w2_scale: torch.Tensor | None = None,
                         apply_router_weight_on_input=False, stream=None, weight_layout=MOE_LAYOUT_ROWS,
                         chunk_tokens: int = 0) -> torch.Tensor:
    """fused_experts with the library's static scratch (64 MiB per GPU) instead of a
    workspace, for callers that cannot allocate: `out` [M, H] bf16 is required (this call
    allocates nothing). Raises MoeError (workspace too small) when the problem needs more
    scratch than that."""
    p = _layer_problem(x, w13, w2, topk_ids, topk_weights, block_m, w13_scale, w2_scale,
                       apply_router_weight_on_input, weight_layout, None, chunk_tokens, "fused_experts_static")
    _need_size(out, _BF, p.M * p.H, "out")
    _check(lib().fused_experts_static(ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                      _ptr(w2_scale), _ptr(topk_ids), _ptr(topk_weights), _ptr(out),
                                      _stream(stream)),
           "fused_experts_static")
    return out


# ------------------------------------------------------------------ stages ---

def moe_expert_gemm(p: MoeProblem, which: int, a: torch.Tensor, w: torch.Tensor,
                    sorted_token_ids: torch.Tensor | None, expert_ids: torch.Tensor,
                    num_tokens_post_padded: torch.Tensor, c: torch.Tensor,
                    a_scale: torch.Tensor | None = None, w_scale: torch.Tensor | None = None,
                    stream=None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped expert GEMM over the aligned layout (which = 1: x.w13^T, 2: z.w2^T).

    workspace (from gemm_workspace_for) enables the split-K tail of the second GEMM, as
    fused_experts runs it."""
    w4 = p.wdtype == MOE_W_W4A8_MXFP4  # E2M1 weights, two per byte
    fp8 = p.wdtype in (MOE_W_FP8_E4M3_BLOCK128, MOE_W_MXFP8) or w4
    mx = p.wdtype == MOE_W_MXFP8       # activation scales: packed E8M0 words (int32)
    cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    N, K = (2 * p.I, p.H) if which == 1 else (p.H, p.I)
    _need_size(a, _F8 if fp8 else _BF, (p.M if which == 1 else cap) * K, "a")
    _need_size(w, _F8 if fp8 else _BF, p.E * N * K // (2 if w4 else 1), "w")
    _need_size(expert_ids, _I32T, cap // p.block_m, "expert_ids")
    _need_size(num_tokens_post_padded, _I32T, 1, "num_tokens_post_padded")
    _need_size(c, _BF, cap * N, "c")
    if which == 1:
        _need_size(sorted_token_ids, _I32T, cap, "sorted_token_ids")
    if fp8:
        _need_size(a_scale, _I32T if mx else _F32, (K // 128) * cap, "a_scale [K/128, cap]")
        _need_size(w_scale, _I32T if (mx or w4) else _F32, p.E * (N if (mx or w4) else N // 128) * (K // 128),
                   "w_scale")
    _check(lib().moe_expert_gemm(ctypes.byref(p), which, _ptr(a), _ptr(a_scale), _ptr(w),
                                 _ptr(w_scale), _ptr(sorted_token_ids), _ptr(expert_ids),
                                 _ptr(num_tokens_post_padded), _ptr(c), _ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream(stream)),
           "moe_expert_gemm")
    return c


def gemm_workspace_for(p: MoeProblem, device="cuda") -> torch.Tensor | None:
    """A workspace for moe_expert_gemm (None if the configuration uses none)."""
    n = lib().moe_expert_gemm_workspace_bytes(ctypes.byref(p))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def moe_silu_and_mul(p: MoeProblem, h: torch.Tensor, sorted_token_ids: torch.Tensor,
                     topk_weights: torch.Tensor, num_tokens_post_padded: torch.Tensor,
                     z: torch.Tensor, z_scale: torch.Tensor | None = None, stream=None):
    fp8 = p.wdtype == MOE_W_FP8_E4M3_BLOCK128
    cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    _need_size(h, _BF, cap * 2 * p.I, "h")
    _need_size(sorted_token_ids, _I32T, cap, "sorted_token_ids")
    _need_size(topk_weights, _F32, p.M * p.topk, "topk_weights")
    _need_size(num_tokens_post_padded, _I32T, 1, "num_tokens_post_padded")
    _need_size(z, _F8 if fp8 else _BF, cap * p.I, "z")
    if fp8:
        _need_size(z_scale, _F32, (p.I // 128) * cap, "z_scale [I/128, cap]")
    _check(lib().moe_silu_and_mul(ctypes.byref(p), _ptr(h), _ptr(sorted_token_ids),
                                  _ptr(topk_weights), _ptr(num_tokens_post_padded), _ptr(z),
                                  _ptr(z_scale), _stream(stream)), "moe_silu_and_mul")
    return z, z_scale


def moe_expert_gemm_act_supported(p: MoeProblem) -> bool:
    return bool(lib().moe_expert_gemm_act_supported(ctypes.byref(p)))


def moe_expert_gemm_act(p: MoeProblem, x: torch.Tensor, x_scale: torch.Tensor | None,
                        w13: torch.Tensor, w13_scale: torch.Tensor | None,
                        sorted_token_ids: torch.Tensor, expert_ids: torch.Tensor,
                        num_tokens_post_padded: torch.Tensor, topk_weights: torch.Tensor,
                        z: torch.Tensor, z_scale: torch.Tensor | None = None, stream=None):
    """GEMM1 with SiLU-and-mul fused in its epilogue -> (z, z_scale).

    bf16 weights (block_m 128 or 256): z [cap, I] bf16, the scales are unused.
    fp8 weights (block_m 128): z [cap, I] e4m3 with z_scale [I/128, cap]."""
    w4 = p.wdtype == MOE_W_W4A8_MXFP4
    fp8 = p.wdtype in (MOE_W_FP8_E4M3_BLOCK128, MOE_W_MXFP8) or w4
    mx = p.wdtype == MOE_W_MXFP8
    cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    _need_size(x, _F8 if fp8 else _BF, p.M * p.H, "x")
    _need_size(w13, _F8 if fp8 else _BF, p.E * 2 * p.I * p.H // (2 if w4 else 1), "w13")
    _need_size(sorted_token_ids, _I32T, cap, "sorted_token_ids")
    _need_size(expert_ids, _I32T, cap // p.block_m, "expert_ids")
    _need_size(num_tokens_post_padded, _I32T, 1, "num_tokens_post_padded")
    _need_size(topk_weights, _F32, p.M * p.topk, "topk_weights")
    _need_size(z, _F8 if fp8 else _BF, cap * p.I, "z")
    if fp8:
        sd = _I32T if mx else _F32
        _need_size(x_scale, sd, (p.H // 128) * cap, "x_scale [H/128, cap]")
        _need_size(w13_scale, _I32T if (mx or w4) else _F32,
                   p.E * (2 * p.I if (mx or w4) else 2 * p.I // 128) * (p.H // 128), "w13_scale")
        _need_size(z_scale, sd, (p.I // 128) * cap, "z_scale [I/128, cap]")
    _check(lib().moe_expert_gemm_act(ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(w13),
                                     _ptr(w13_scale), _ptr(sorted_token_ids), _ptr(expert_ids),
                                     _ptr(num_tokens_post_padded), _ptr(topk_weights), _ptr(z),
                                     _ptr(z_scale), _stream(stream)), "moe_expert_gemm_act")
    return z, z_scale


def moe_permute_scales(p: MoeProblem, scale: torch.Tensor, sorted_token_ids: torch.Tensor,
                       num_tokens_post_padded: torch.Tensor, out: torch.Tensor, stream=None):
    """Per-token fp8 group scales [M, H/128] -> group-major, sorted-order [H/128, cap]; MXFP8:
    the [M, H/32] E8M0 bytes as [M, H/128] int32 words (4 blocks each), moved the same way."""
    cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    _need_size(scale, (torch.float32, torch.int32), p.M * (p.H // 128), "scale")
    _need_size(sorted_token_ids, _I32T, cap, "sorted_token_ids")
    _need_size(num_tokens_post_padded, _I32T, 1, "num_tokens_post_padded")
    _need_size(out, (torch.float32, torch.int32), (p.H // 128) * cap, "out [H/128, cap]")
    _check(lib().moe_permute_scales(ctypes.byref(p), _ptr(scale), _ptr(sorted_token_ids),
                                    _ptr(num_tokens_post_padded), _ptr(out), _stream(stream)),
           "moe_permute_scales")
    return out


def moe_unpermute_reduce(p: MoeProblem, o: torch.Tensor, inv_perm: torch.Tensor,
                         topk_weights: torch.Tensor, y: torch.Tensor, stream=None):
    cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m)
    _need_size(o, _BF, cap * p.H, "o")
    _need_size(inv_perm, _I32T, p.M * p.topk, "inv_perm")
    _need_size(topk_weights, _F32, p.M * p.topk, "topk_weights")
    _need_size(y, _BF, p.M * p.H, "y")
    _check(lib().moe_unpermute_reduce(ctypes.byref(p), _ptr(o), _ptr(inv_perm),
                                      _ptr(topk_weights), _ptr(y), _stream(stream)),
           "moe_unpermute_reduce")
    return y


def moe_pack_weights(p: MoeProblem, which: int, w: torch.Tensor, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Rewrite bf16 w13 (which = 1, [E, 2I, H]) or w2 (which = 2, [E, H, I]) into the
    MOE_LAYOUT_TILED element order (16 x 32 tiles); the result has the same shape and bytes."""
    N, K = (2 * p.I, p.H) if which == 1 else (p.H, p.I)
    _need_size(w, _BF, p.E * N * K, "w")
    if out is None:
        out = torch.empty_like(w)
    _need_size(out, _BF, p.E * N * K, "out")
    _check(lib().moe_pack_weights(ctypes.byref(p), which, _ptr(w), _ptr(out), _stream(stream)),
           "moe_pack_weights")
    return out


def moe_batched_experts(a: torch.Tensor, expert_num_tokens: torch.Tensor, w13: torch.Tensor,
                        w2: torch.Tensor, block_m: int, w13_scale: torch.Tensor | None = None,
                        w2_scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None,
                        weight_layout=MOE_LAYOUT_ROWS) -> torch.Tensor:
    """Batched-experts form: a [E, max_M, H] bf16 (one batch per expert), expert_num_tokens
    [E] int32 -> out [E, max_M, H] bf16, rows past a count 0, unweighted."""
    _need(a, torch.bfloat16, "a")
    _need(expert_num_tokens, torch.int32, "expert_num_tokens")
    fp8 = w13.dtype == torch.float8_e4m3fn
    wdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    _need(w13, wdt, "w13")
    _need(w2, wdt, "w2")
    E, max_M, H = a.shape
    E2, N2, H2 = w13.shape
    if E2 != E or H2 != H or tuple(w2.shape) != (E, H, N2 // 2) or expert_num_tokens.numel() != E:
        raise ValueError("moe_batched_experts: inconsistent shapes")
    if fp8:
        _need(w13_scale, torch.float32, "w13_scale")
        _need(w2_scale, torch.float32, "w2_scale")
    p = make_problem(max_M, H, N2 // 2, E, 1, block_m,
                     MOE_W_FP8_E4M3_BLOCK128 if fp8 else MOE_W_BF16, False, weight_layout)
    check_weight_scales(p.wdtype, E, H, N2 // 2, w13_scale, w2_scale, "moe_batched_experts")
    if out is None:
        out = torch.empty_like(a)
    _need(out, torch.bfloat16, "out")
    if workspace is None:
        n = moe_batched_workspace_bytes(p)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=a.device)
    _check(lib().moe_batched_experts(ctypes.byref(p), _ptr(a), _ptr(expert_num_tokens), _ptr(w13),
                                     _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_batched_experts")
    return out


def moe_batched_workspace_bytes(p: MoeProblem) -> int:
    return int(lib().moe_batched_workspace_bytes(ctypes.byref(p)))


def moe_quant_mx_groups(x: torch.Tensor, stream=None):
    """MXFP8 quantisation per 32 columns -> (q e4m3 [rows, cols], scale uint8 E8M0 [rows, cols/32])."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quant_mx_groups(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(stream)),
           "moe_quant_mx_groups")
    return q, s


def moe_pack_mx_scales(p: MoeProblem, which: int, scale: torch.Tensor, stream=None) -> torch.Tensor:
    """MXFP8 weight scales [E, N, K/32] uint8 -> packed words [E, K/128, N] int32."""
    N, K = (2 * p.I, p.H) if which == 1 else (p.H, p.I)
    _need_size(scale, (torch.uint8,), p.E * N * (K // 32), "scale")
    out = torch.empty((p.E, K // 128, N), dtype=torch.int32, device=scale.device)
    _check(lib().moe_pack_mx_scales(ctypes.byref(p), which, _ptr(scale), _ptr(out), _stream(stream)),
           "moe_pack_mx_scales")
    return out
