#!/usr/bin/env python3
"""Throughput of the fused MoE expert forward on one MI355X.

A step is one pass of the whole hot path over one batch: the router
(moe_topk) and fused_experts (align, GEMM1, SiLU-and-mul, GEMM2, weighted
unpermute-reduce; fp8 adds the activation quantisation). Inputs are seeded,
synthetic and resident in HBM before the timed region starts.

Printed JSON line (rank 0):
  value        whole-job algorithmic TFLOP/s (6*M*topk*H*I per step); tokens/s beside it
  roofline     the dominant kernel (GEMM1): algorithmic FLOP or bytes per launch divided
               by its average duration, from HIP events recorded on its stream over a
               second timed region that launches the same kernels stage by stage
  cpu_baseline the CPU oracle timed on a bounded sample of tokens of the same workload
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402

METRIC = "fused-MoE layer TFLOP/s and tokens/s at 1 MI355X; % of MFMA or HBM roofline"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0                           # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("gemm.hip", "gemm_stream.hip", "layout.h", "common.h", "kernels.h", "api.hip")


def kernel_source_digest() -> str:
    """sha256 over the GEMM sources; a traffic measurement is only reported for the
    kernel it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_ffn_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_block_m(kernel: str) -> int:
    """Row-block size of a GEMM kernel from its name in a profile: the first template
    argument of the tile configuration, or 16 for the weight-streaming kernel."""
    if "Cfg<" in kernel:
        return int(kernel.split("Cfg<", 1)[1].split(",", 1)[0])
    return 16 if "stream_gemm" in kernel else -1


def read_profile(path: str, block_m: int):
    """key = value lines of a committed counter profile, or None if there is none, the
    kernel sources changed since it was taken, or it was taken with another block_m."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_digest():
        return None
    if profile_block_m(kv.get("kernel", "")) != block_m:
        return None
    return kv


def measured_traffic(workload: str, block_m: int):
    """HBM bytes per GEMM1 launch from the committed counter profile of this workload
    (FETCH_SIZE + WRITE_SIZE, each scaled by a copy kernel of known size), or None."""
    kv = read_profile(os.path.join(PROFILES, f"gemm1_{workload}_traffic.txt"), block_m)
    return None if kv is None else float(kv["hbm_bytes_per_launch"].split()[0])


def measured_mfma(workload: str, block_m: int):
    """MFMA-busy fraction of the SIMDs and the clock during GEMM1 from the committed
    counter profile of this workload (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE), or None."""
    kv = read_profile(os.path.join(PROFILES, f"gemm1_{workload}_mfma.txt"), block_m)
    if kv is None:
        return None
    return {"busy_fraction": float(kv["mfma_busy_fraction"].split()[0]),
            "clock_ghz": float(kv["clock_ghz"].split()[0])}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    # the default is the largest single-GPU configuration: the DeepSeek-V3-shaped prefill
    # with skewed routing (8192 tokens, 256 experts, top-8; 5.77 TFLOP per step)
    ap.add_argument("--workload", default="dsv3_skewed_prefill_m8192", choices=list(synth.WORKLOADS))
    ap.add_argument("--block-m", type=int, default=None, help="override the workload's block_m")
    ap.add_argument("--weight-layout", default="auto", choices=("auto", "rows", "tiled"),
                    help="element order of w13/w2: auto = the tiled order where the library "
                         "supports it (bf16 with block_m 16, 128 or 256), else row-major")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the timed region, so "
                         "that a counter profile of this command can scale FETCH_SIZE and "
                         "WRITE_SIZE by a kernel whose traffic is known")
    return ap.parse_args()


class Step:
    """Device buffers and the two ways of running one step."""

    def __init__(self, p: synth.Problem, d: synth.Inputs, layout: str = "auto", weights=None):
        import mixture_experts_ffn_block_amd as moe
        self.moe, self.p, self.d = moe, p, d
        self.fp8 = p.wdtype in ("fp8", "mxfp8", "w4a8")  # 8-bit activations
        self.mx = p.wdtype == "mxfp8"                     # E8M0 scales per 32 on both operands
        self.w4 = p.wdtype == "w4a8"                      # E2M1 weights with E8M0 scales
        dev = d.x.device
        # an expert-parallel rank holds E / ep_size experts; ids stay global
        self.emap = d.expert_map
        G = p.E if self.emap is not None else 0
        M, H, I, E, k, B = p.M, p.H, p.I, len(p.local_experts), p.topk, p.block_m
        wdt = (moe.MOE_W_MXFP8 if self.mx else moe.MOE_W_W4A8_MXFP4 if self.w4
               else moe.MOE_W_FP8_E4M3_BLOCK128 if self.fp8 else moe.MOE_W_BF16)
        rows = moe.make_problem(M, H, I, E, k, B, wdt, p.apply_router_weight_on_input)
        packable = not self.fp8 and B in (16, 128, 256)
        if layout == "tiled" and not packable:
            raise SystemExit("--weight-layout tiled needs bf16 weights and block_m 16, 128 or 256")
        self.layout = "tiled" if packable and layout in ("auto", "tiled") else "rows"
        self.wl = moe.MOE_LAYOUT_TILED if self.layout == "tiled" else moe.MOE_LAYOUT_ROWS
        self.prob = moe.make_problem(M, H, I, E, k, B, wdt, p.apply_router_weight_on_input, self.wl, G)
        self.ids = torch.empty((M, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((M, k), dtype=torch.float32, device=dev)
        self.y = torch.empty_like(d.x)
        self.ws = moe.workspace_for(self.prob, dev)
        cap = moe.moe_align_capacity(M, k, E, B)
        self.cap = cap
        # buffers of the staged run
        i32 = dict(dtype=torch.int32, device=dev)
        self.sorted = torch.empty(cap, **i32)
        self.expert_ids = torch.empty(cap // B, **i32)
        self.npp = torch.zeros(1, **i32)
        self.inv = torch.empty((M, k), **i32)
        self.h = torch.empty((cap, 2 * I), dtype=torch.bfloat16, device=dev)
        self.o = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        adt = torch.float8_e4m3fn if self.fp8 else torch.bfloat16
        self.z = torch.empty((cap, I), dtype=adt, device=dev)
        sdt = torch.int32 if self.mx else torch.float32  # MX: four E8M0 bytes per word
        self.zs = torch.empty((I // 128, cap), dtype=sdt, device=dev) if self.fp8 else None
        if self.fp8:
            self.xq = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
            self.xs = torch.empty((M, H // 128), dtype=sdt, device=dev)
            self.xst = torch.empty((H // 128, cap), dtype=sdt, device=dev)
        self.act_fused = moe.moe_expert_gemm_act_supported(self.prob)
        self.gws = moe.gemm_workspace_for(self.prob, dev)  # split-K tail of the second GEMM
        self.w13 = d.w13q if self.fp8 else d.w13
        self.w2 = d.w2q if self.fp8 else d.w2
        self.w13s, self.w2s = d.w13s, d.w2s
        if self.mx or self.w4:  # weight-scale preparation, once, outside every timed region
            self.w13s = moe.moe_pack_mx_scales(rows, 1, d.w13s)
            self.w2s = moe.moe_pack_mx_scales(rows, 2, d.w2s)
        if weights is not None:  # prepared by another Step of the same workload
            self.w13, self.w2 = weights
        elif self.layout == "tiled":  # weight preparation, once, outside every timed region
            self.w13 = moe.moe_pack_weights(rows, 1, d.w13)
            self.w2 = moe.moe_pack_weights(rows, 2, d.w2)

    def route(self):
        """The workload's router: softmax top-k, or the grouped / sigmoid router."""
        m, d, p = self.moe, self.d, self.p
        if p.scoring == "softmax" and p.n_group == 1 and d.score_bias is None and p.routed_scale == 1.0:
            m.moe_topk(d.logits, p.topk, out=(self.ids, self.w))
        else:
            m.moe_topk_grouped(d.logits, p.topk, p.scoring, True, p.n_group, p.topk_group, d.score_bias,
                               p.routed_scale, out=(self.ids, self.w))

    def fused(self):
        self.route()
        self.experts()

    def experts(self):
        """fused_experts alone, on the router's last ids and weights."""
        m, d = self.moe, self.d
        m.fused_experts(d.x, self.w13, self.w2, self.ids, self.w, self.p.block_m,
                        self.w13s, self.w2s, self.p.apply_router_weight_on_input, out=self.y,
                        workspace=self.ws, weight_layout=self.wl, expert_map=self.emap,
                        chunk_tokens=self.p.chunk_tokens)

    STAGES = ("router", "quant", "align", "gemm1", "act", "gemm2", "reduce")

    def staged(self, ev):
        """The same kernels, launched stage by stage; ev[i] is recorded after stage i."""
        m, d, p = self.moe, self.d, self.prob
        lib = m.lib()
        s = m._stream()
        ev[0].record()
        self.route()
        ev[1].record()
        a1, a1s = d.x, None
        if self.fp8:
            quant = lib.moe_quant_mx_groups if self.mx else lib.moe_quant_fp8_groups
            quant(m._ptr(d.x), self.p.M, self.p.H, m._ptr(self.xq), m._ptr(self.xs), s)
            a1, a1s = self.xq, self.xst
        ev[2].record()
        if self.emap is None:
            lib.moe_align_block_size(m._ptr(self.ids), self.p.M, self.p.topk, self.p.E,
                                     self.p.block_m, m._ptr(self.sorted), m._ptr(self.expert_ids),
                                     m._ptr(self.npp), m._ptr(self.inv), s)
        else:
            lib.moe_align_block_size_ep(m._ptr(self.ids), self.p.M, self.p.topk, self.p.E,
                                        m._ptr(self.emap), p.E, self.p.block_m, m._ptr(self.sorted),
                                        m._ptr(self.expert_ids), m._ptr(self.npp), m._ptr(self.inv), s)
        if self.fp8:  # the activation scales follow the rows into the sorted order
            m.moe_permute_scales(p, self.xs, self.sorted, self.npp, self.xst)
        ev[3].record()
        if self.act_fused:  # GEMM1 with the activation in its epilogue; no separate act stage
            m.moe_expert_gemm_act(p, a1, a1s, self.w13, self.w13s, self.sorted, self.expert_ids,
                                  self.npp, self.w, self.z, self.zs)
            ev[4].record()
        else:
            m.moe_expert_gemm(p, 1, a1, self.w13, self.sorted, self.expert_ids, self.npp, self.h,
                              a1s, self.w13s)
            ev[4].record()
            m.moe_silu_and_mul(p, self.h, self.sorted, self.w, self.npp, self.z, self.zs)
        ev[5].record()
        m.moe_expert_gemm(p, 2, self.z, self.w2, None, self.expert_ids, self.npp, self.o,
                          self.zs, self.w2s, workspace=self.gws)
        ev[6].record()
        m.moe_unpermute_reduce(p, self.o, self.inv, self.w, self.y)
        ev[7].record()


class BatchedStep(Step):
    """The batched-experts form: the router's items of the workload, presented as one
    batch of up to M rows per expert (built once, outside every timed region, as a
    low-latency dispatch would deliver them), then moe_batched_experts. The staged
    run launches the same kernels as the equivalent top-1 routed problem over the
    E * M batch rows."""

    STAGES = Step.STAGES

    def __init__(self, p: synth.Problem, d: synth.Inputs, layout: str = "auto"):
        super().__init__(p, d, layout)
        if self.fp8 or self.emap is not None:
            raise SystemExit("the batched workload is bf16 on all experts")
        m, dev = self.moe, d.x.device
        E, M, k, H, I, B = p.E, p.M, p.topk, p.H, p.I, p.block_m
        self.route()
        flat = self.ids.reshape(-1).long()
        order = torch.argsort(flat, stable=True)            # items by expert, tokens ascending
        counts = torch.bincount(flat, minlength=E)
        e_sorted = flat[order]
        pos = torch.arange(flat.numel(), device=dev) - (torch.cumsum(counts, 0) - counts)[e_sorted]
        self.a = torch.zeros((E, M, H), dtype=torch.bfloat16, device=dev)
        self.a[e_sorted, pos] = d.x[order // k]
        self.counts = counts.to(torch.int32)
        self.out = torch.empty_like(self.a)
        self.pb = m.make_problem(M, H, I, E, 1, B, m.MOE_W_BF16, False, self.wl)
        self.bws = torch.empty(max(m.moe_batched_workspace_bytes(self.pb), 256), dtype=torch.uint8,
                               device=dev)
        # the equivalent routed top-1 problem, for the staged run
        r = torch.arange(M, device=dev)
        self.qids = torch.where(r[None, :] < counts[:, None], torch.arange(E, device=dev)[:, None],
                                torch.full_like(r[None, :], -1)).to(torch.int32).reshape(E * M, 1).contiguous()
        self.q = m.make_problem(E * M, H, I, E, 1, B, m.MOE_W_BF16, False, self.wl)
        cap = m.moe_align_capacity(E * M, 1, E, B)
        i32 = dict(dtype=torch.int32, device=dev)
        self.sorted_q = torch.empty(cap, **i32)
        self.expert_ids_q = torch.empty(cap // B, **i32)
        self.npp_q = torch.zeros(1, **i32)
        self.inv_q = torch.empty((E * M, 1), **i32)
        self.z_q = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
        self.h_q = torch.empty((cap, 2 * I), dtype=torch.bfloat16, device=dev)
        self.o_q = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        self.ones_q = torch.ones((E * M, 1), dtype=torch.float32, device=dev)
        self.act_fused = m.moe_expert_gemm_act_supported(self.q)
        self.gws = m.gemm_workspace_for(self.q, dev)

    def fused(self):
        self.moe.moe_batched_experts(self.a, self.counts, self.w13, self.w2, self.p.block_m,
                                     out=self.out, workspace=self.bws, weight_layout=self.wl)

    def experts(self):
        self.fused()

    def staged(self, ev):
        m, q = self.moe, self.q
        E, M = self.p.E, self.p.M
        a = self.a.view(E * M, self.p.H)
        ev[0].record()
        ev[1].record()
        ev[2].record()
        m.lib().moe_align_block_size(m._ptr(self.qids), E * M, 1, E, self.p.block_m, m._ptr(self.sorted_q),
                                     m._ptr(self.expert_ids_q), m._ptr(self.npp_q), m._ptr(self.inv_q),
                                     m._stream())
        ev[3].record()
        if self.act_fused:
            m.moe_expert_gemm_act(q, a, None, self.w13, None, self.sorted_q, self.expert_ids_q, self.npp_q,
                                  self.ones_q, self.z_q)
            ev[4].record()
        else:
            m.moe_expert_gemm(q, 1, a, self.w13, self.sorted_q, self.expert_ids_q, self.npp_q, self.h_q)
            ev[4].record()
            m.moe_silu_and_mul(q, self.h_q, self.sorted_q, self.ones_q, self.npp_q, self.z_q)
        ev[5].record()
        m.moe_expert_gemm(q, 2, self.z_q, self.w2, None, self.expert_ids_q, self.npp_q, self.o_q,
                          workspace=self.gws)
        ev[6].record()
        m.moe_unpermute_reduce(q, self.o_q, self.inv_q, self.ones_q, self.out.view(E * M, self.p.H))
        ev[7].record()


def algorithmic(p: synth.Problem, touched: int, act_fused: bool = False, R: int | None = None):
    """Algorithmic FLOP and HBM bytes of the step and of GEMM1 (padding excluded);
    with the activation fused into GEMM1 that kernel writes z instead of h. R: the
    routed items computed here (all M * topk, or an expert-parallel rank's share)."""
    R = p.M * p.topk if R is None else R
    q8 = p.wdtype in ("fp8", "mxfp8", "w4a8")
    ab = 1 if q8 else 2                            # activation bytes per value
    wb = 0.5 if p.wdtype == "w4a8" else ab         # weight bytes per value
    # scale bytes per K value: fp32 per 128x128 block (weights) or per 128 (activations),
    # or one E8M0 byte per 32 values (MX weights; MXFP8 activations)
    ws_per = 1.0 / 32 if p.wdtype in ("mxfp8", "w4a8") else 4.0 / (128 * 128)
    as_per = 1.0 / 32 if p.wdtype == "mxfp8" else 4.0 / 128
    flops_g1 = 4.0 * R * p.H * p.I
    flops = 6.0 * R * p.H * p.I
    w13_b = touched * 2 * p.I * p.H * wb
    w2_b = touched * p.H * p.I * wb
    if q8:
        w13_b += touched * 2 * p.I * p.H * ws_per
        w2_b += touched * p.H * p.I * ws_per
    x_b = p.M * p.H * 2
    y_b = p.M * p.H * 2
    logits_b = p.M * p.E * 4
    xin_g1 = p.M * p.H * ab + (p.M * p.H * as_per if q8 else 0)
    if act_fused:
        out_g1 = R * p.I * ab + (R * p.I * as_per if q8 else 0)
    else:
        out_g1 = R * 2 * p.I * 2
    return dict(flops=flops, bytes=w13_b + w2_b + x_b + y_b + logits_b,
                flops_g1=flops_g1, bytes_g1=w13_b + xin_g1 + out_g1)


def stage_work(p: synth.Problem, touched: int, R: int, npp: int, act_fused: bool):
    """Algorithmic HBM bytes (and FLOP for the GEMMs) of each stage of one step: what the
    stage must read and write at least, padding rows counted only where a stage writes
    them (align's layout, the per-row activation outputs)."""
    q8 = p.wdtype in ("fp8", "mxfp8", "w4a8")
    ab = 1 if q8 else 2
    wb = 0.5 if p.wdtype == "w4a8" else ab
    a_sc = 1.0 / 32 if p.wdtype == "mxfp8" else 4.0 / 128       # activation scale bytes per value
    w_sc = 1.0 / 32 if p.wdtype in ("mxfp8", "w4a8") else 4.0 / (128 * 128)
    M, H, I, E, k = p.M, p.H, p.I, p.E, p.topk
    w = {}
    w["router"] = {"bytes": M * E * 4 + M * k * 8}
    if q8:
        w["quant"] = {"bytes": M * H * 2 + M * H + M * H * a_sc}
    # align: ids in; sorted ids, block experts, inv_perm out (+ the activation scales'
    # permute on the 8-bit paths)
    w["align"] = {"bytes": R * 4 + npp * 4 + npp // p.block_m * 4 + R * 4
                  + ((M * H * a_sc + npp * H * a_sc) if q8 else 0)}
    z_b = npp * I * ab + (npp * I * a_sc if q8 else 0)
    w13 = touched * 2 * I * H * (wb + (w_sc if q8 else 0))
    w2 = touched * H * I * (wb + (w_sc if q8 else 0))
    x_in = M * H * ab + (M * H * a_sc if q8 else 0)
    if act_fused:
        w["gemm1"] = {"flops": 4.0 * R * H * I, "bytes": w13 + x_in + z_b}
    else:
        w["gemm1"] = {"flops": 4.0 * R * H * I, "bytes": w13 + x_in + npp * 2 * I * 2}
        w["act"] = {"bytes": npp * 2 * I * 2 + z_b}
    w["gemm2"] = {"flops": 2.0 * R * H * I, "bytes": w2 + z_b + npp * H * 2}
    w["reduce"] = {"bytes": R * H * 2 + R * 4 + M * H * 2}
    return w


def stage_roofline(work: dict, stage_ms: dict, dt: str) -> dict:
    """Each stage's achieved rate against its binding roofline (the larger of its FLOP
    and byte times at the spec peaks). A stage whose roofline time is under 2 us is
    bound by launch and dependency latency, not by either peak: it reports its time."""
    out = {}
    for name, wk in work.items():
        ms = stage_ms.get(name, 0.0)
        if ms <= 0:
            continue
        t = ms * 1e-3
        t_hbm = wk["bytes"] / (PEAK_HBM_GBS * 1e9)
        t_mfma = wk.get("flops", 0.0) / (PEAK_TFLOPS[dt] * 1e12)
        if max(t_hbm, t_mfma) < 2e-6:
            out[name] = {"bound": "latency", "us": round(ms * 1e3, 1), "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 2)}
        elif t_mfma > t_hbm:
            out[name] = {"bound": "mfma", "achieved": round(wk["flops"] / t / 1e12, 2), "unit": "TFLOP/s",
                         "frac": round(t_mfma / t, 4)}
        else:
            out[name] = {"bound": "hbm", "achieved": round(wk["bytes"] / t / 1e9, 1), "unit": "GB/s",
                         "frac": round(t_hbm / t, 4)}
    return out


def cpu_model() -> str:
    """The host CPU's model name, its family / model numbers (a virtualised host may
    report only a generic name) and the logical CPU count, from /proc/cpuinfo."""
    try:
        fields: dict = {}
        names = 0
        for l in open("/proc/cpuinfo"):
            key, _, val = l.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name":
                names += 1
            if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = val
        if not names:
            return "unknown"
        ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
        return f"{fields['model name']} ({ids + '; ' if ids else ''}{names} logical CPUs)"
    except OSError:
        return "unknown"


def copy_bandwidth(mib: int = 2048, reps: int = 10) -> dict:
    """Achievable HBM bandwidth on this GPU: a device-to-device copy of `mib` MiB (read
    plus write bytes over the copy's time, HIP events on the current stream), timed
    outside every timed region; the median of `reps` copies."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.median(times))
    del src, dst
    return {"copy_GBs": round(2 * (mib << 20) / t / 1e9, 1), "bytes_per_copy": 2 * (mib << 20),
            "spec_GBs": PEAK_HBM_GBS, "frac_of_spec": round(2 * (mib << 20) / t / 1e9 / PEAK_HBM_GBS, 4),
            "method": f"torch copy_ of {mib} MiB on the device, median of {reps}, read + write bytes"}


def cpu_baseline(p: synth.Problem, d: synth.Inputs, ids: torch.Tensor, w: torch.Tensor,
                 target_s: float):
    """The CPU oracle on a bounded sample of tokens (test infrastructure, timed as a baseline)."""
    import oracle
    threads = oracle.threads()

    def bits16(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def bits8(t):
        return t.cpu().contiguous().view(torch.uint8).numpy()

    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    # experts held here: global id -> row of the weight tensors (an expert-parallel
    # rank holds a slice; other slots are computed elsewhere and skipped)
    held = np.full(p.E, -1, np.int64)
    held[list(p.local_experts)] = np.arange(len(p.local_experts))

    def run(T):
        toks = np.arange(T)
        experts = sorted(e for e in set(ids_np[toks].reshape(-1).tolist()) if held[e] >= 0)
        remap = np.full(p.E, -1, np.int32)
        remap[experts] = np.arange(len(experts), dtype=np.int32)
        sub_ids = ids_np[toks]
        sel = torch.tensor(held[experts], device=d.x.device)
        x = bits16(d.x[:T])
        if p.wdtype in ("mxfp8", "w4a8"):  # (no expert map: every expert is held)
            t0 = time.perf_counter()
            oracle.fused_experts_mx(x, bits8(d.w13q[sel]), d.w13s[sel].cpu().numpy(), bits8(d.w2q[sel]),
                                    d.w2s[sel].cpu().numpy(), remap[sub_ids], w_np[toks],
                                    w4=p.wdtype == "w4a8", on_input=p.apply_router_weight_on_input)
            return time.perf_counter() - t0, int((held[ids_np[toks]] >= 0).sum())
        if p.wdtype == "fp8":
            args = (x, bits8(d.w13q[sel]), d.w13s[sel].cpu().numpy(), bits8(d.w2q[sel]),
                    d.w2s[sel].cpu().numpy(), sub_ids, w_np[toks])
            fn = oracle.fused_experts_fp8
        else:
            args = (x, bits16(d.w13[sel]), bits16(d.w2[sel]), sub_ids, w_np[toks])
            fn = oracle.fused_experts_bf16
        t0 = time.perf_counter()
        fn(*args, on_input=p.apply_router_weight_on_input, expert_map=remap)
        return time.perf_counter() - t0, int((held[ids_np[toks]] >= 0).sum())

    T = min(p.M, threads)
    dt, items = run(T)
    if dt < target_s / 2 and T < p.M:
        T = int(min(p.M, max(T, round(T * target_s / dt / threads) * threads)))
        dt, items = run(T)
    flops = 6.0 * items * p.H * p.I
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "tokens_per_s": round(T / dt, 3), "seconds": round(dt, 3),
            "sample": f"first {T} of {p.M} tokens of the same workload (all their top-{p.topk} "
                      f"experts held here, {items} routed items), plain C oracle, fp64 "
                      f"accumulation, {threads} OpenMP threads"}


def cpu_baseline_batched(p: synth.Problem, d: synth.Inputs, st: "BatchedStep", target_s: float):
    """The CPU oracle of the batched form on the batches of the first experts."""
    import oracle
    threads = oracle.threads()
    bits16 = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    counts = st.counts.cpu().numpy()

    def run(n):
        sel = slice(0, n)
        t0 = time.perf_counter()
        oracle.batched_experts_bf16(bits16(st.a[sel]), counts[sel], bits16(d.w13[sel]), bits16(d.w2[sel]))
        return time.perf_counter() - t0

    n = min(p.E, 4)
    dt = run(n)
    if dt < target_s / 2 and n < p.E:
        n = int(min(p.E, max(n, round(n * target_s / dt))))
        dt = run(n)
    items = int(np.clip(counts[:n], 0, p.M).sum())
    return {"value": round(6.0 * items * p.H * p.I / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "seconds": round(dt, 3),
            "sample": f"the batches of the first {n} of {p.E} experts ({items} rows), plain C oracle, "
                      f"fp64 accumulation, {threads} OpenMP threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1",
                          "gpus_requested": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import mixture_experts_ffn_block_amd as moe
    moe.lib()  # fails loudly if the HIP library is missing

    over = {} if args.block_m is None else {"block_m": args.block_m}
    p = synth.Problem.named(args.workload, **over)
    print(f"# workload {args.workload}: {p}", file=sys.stderr, flush=True)
    d = synth.make_inputs(p, "cuda")
    st = (BatchedStep if p.batched else Step)(p, d, args.weight_layout)
    # a chunked layer launches its kernels once per chunk: the staged breakdown (and the
    # roofline of GEMM1 per launch) runs the first chunk
    chunked = 0 < p.chunk_tokens < p.M
    if chunked:
        pc = dataclasses.replace(p, M=p.chunk_tokens, chunk_tokens=0)
        dc = dataclasses.replace(d, x=d.x[:pc.M], logits=d.logits[:pc.M])
        sst = Step(pc, dc, args.weight_layout, weights=(st.w13, st.w2))
    else:
        pc, sst = p, st
    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    # outside every timed region; a counter run skips it, so that its calibration copy
    # stays the only large device copy the counters see
    hbm = copy_bandwidth() if args.copy_calibration_mib <= 0 else None
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        st.fused()

    # timed region: K steps through the product entry points, one event before and one
    # after, between synchronisations. It follows the warm-up directly: host work here
    # would leave the GPU idle, and after ~10 ms idle its first milliseconds of work run
    # slower (about 3 ms of extra time over the next 20 prefill steps, measured)
    t0_ev, t1_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    t0_ev.record()
    for _ in range(args.steps):
        st.fused()
    t1_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = t0_ev.elapsed_time(t1_ev) / args.steps
    # each step's own duration: K more steps with an event between steps (not
    # synchronising; a recorded event costs the stream a few microseconds, which
    # these durations include and the timed region above does not)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        st.fused()
        marks[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    # fused_experts alone (the router's output already in place), K calls
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for _ in range(args.steps):
        st.experts()
    b_ev.record()
    torch.cuda.synchronize()
    ms_experts = a_ev.elapsed_time(b_ev) / args.steps

    # stage breakdown: the same kernels stage by stage, HIP events on the same stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    for _ in range(2):
        sst.staged([torch.cuda.Event(enable_timing=True) for _ in range(8)])
    torch.cuda.synchronize()
    for i in range(args.steps):
        sst.staged(evs[i])
    torch.cuda.synchronize()
    ids_host = st.ids.cpu().numpy()
    # experts touched and routed items computed here (an expert-parallel rank: its share)
    held = np.zeros(p.E, bool)
    held[list(p.local_experts)] = True
    touched = int(np.unique(ids_host[held[ids_host]]).size)
    items = int(held[ids_host].sum())
    ids_stage = sst.ids.cpu().numpy()
    alg_stage = algorithmic(pc, int(np.unique(ids_stage[held[ids_stage]]).size), sst.act_fused,
                            int(held[ids_stage].sum()))
    stage_ms = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
                for j, name in enumerate(Step.STAGES)}
    staged_total = float(np.mean([e[0].elapsed_time(e[7]) for e in evs]))

    touched_stage, items_stage = int(np.unique(ids_stage[held[ids_stage]]).size), int(held[ids_stage].sum())
    if p.batched:  # the staged run is the top-1 problem over the E * M batch rows; no router
        work = stage_work(dataclasses.replace(pc, M=p.E * p.M, topk=1), touched_stage, items_stage,
                          int(sst.npp_q.item()), sst.act_fused)
        del work["router"]
    else:
        work = stage_work(pc, touched_stage, items_stage, int(sst.npp.item()), sst.act_fused)
    # only the stages that launch kernels (no fp8 quantiser on bf16, no separate act
    # where GEMM1 carries it); an empty interval between two events is reported beside
    # them, since every stage's interval includes it
    stage_ms = {k: v for k, v in stage_ms.items() if k in work}
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in pairs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    empty_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))

    alg = algorithmic(p, touched, st.act_fused, items)
    tflops = alg["flops"] / (ms * 1e-3) / 1e12
    tok_s = p.M / (ms * 1e-3)
    dt = "fp8" if p.wdtype in ("fp8", "mxfp8", "w4a8") else "bf16"
    g1_s = stage_ms["gemm1"] * 1e-3
    t_mfma = alg_stage["flops_g1"] / (PEAK_TFLOPS[dt] * 1e12)
    t_hbm = alg_stage["bytes_g1"] / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(alg_stage["flops_g1"] / g1_s / 1e12, 2),
                "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg_stage["bytes_g1"] / g1_s / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(args.workload, p.block_m)
    if roof["bound"] == "mfma":
        # counters: the share of SIMD cycles the matrix cores were busy, and the clock
        # (the chip is power-limited, so the spec peak at 2.4 GHz is not reached)
        roof["mfma_counters"] = measured_mfma(args.workload, p.block_m)
    roof["kernel"] = ("gemm1 + SiLU-and-mul epilogue (grouped expert GEMM, gathered token rows x w13, writes z)"
                      if st.act_fused else "gemm1 (grouped expert GEMM, gathered token rows x w13)")
    roof["avg_ms"] = round(stage_ms["gemm1"], 4)
    t_star = max(alg["flops"] / (PEAK_TFLOPS[dt] * 1e12), alg["bytes"] / (PEAK_HBM_GBS * 1e9))

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s",
        "tokens_per_s": round(tok_s, 1), "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"mxfp8": "mxfp8", "w4a8": "fp4 x fp8"}.get(p.wdtype, dt),
        "data": "synthetic",
        "config": {"workload": args.workload, "M": p.M, "H": p.H, "I": p.I, "E": p.E,
                   "topk": p.topk, "block_m": p.block_m, "weights": p.wdtype,
                   "weight_layout": st.layout,
                   "experts_touched": touched, "seed": p.seed,
                   **({"ep_size": p.ep_size, "ep_rank": p.ep_rank, "experts_held": len(p.local_experts),
                       "routed_items_here": items} if p.ep_size > 1 else {}),
                   **({"form": "batched experts [E, M, H] (the timed step is moe_batched_experts; "
                               "router and dispatch precede it)", "batch_rows_max": p.M}
                      if p.batched else {}),
                   **({"chunk_tokens": p.chunk_tokens, "stage_scope": f"first chunk of {pc.M} tokens"}
                      if chunked else {})},
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "step_roofline_frac": round(t_star / (ms * 1e-3), 4),
        # the step's algorithmic FLOP and bytes against the spec peaks, each on its own
        "step_fractions": {"mfma": round(alg["flops"] / (PEAK_TFLOPS[dt] * 1e12) / (ms * 1e-3), 4),
                           "hbm_algorithmic": round(alg["bytes"] / (PEAK_HBM_GBS * 1e9) / (ms * 1e-3), 4)},
        "step_bytes_algorithmic": int(alg["bytes"]),
        "ms_fused_experts": round(ms_experts, 4),
        "roofline": roof,
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_roofline": stage_roofline(work, stage_ms, dt),
        "staged_ms_per_step": round(staged_total, 4),
        # as built: what the staged kernels read and write at least, intermediates included
        "staged_bytes_as_built": int(sum(w["bytes"] for w in work.values())),
        "staged_hbm_frac_as_built": round(sum(w["bytes"] for w in work.values()) / (PEAK_HBM_GBS * 1e9)
                                          / (staged_total * 1e-3), 4),
        "empty_event_interval_ms": round(empty_ms, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "hbm_measured": hbm,
    }
    if args.cpu_seconds > 0:
        print("# timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = (cpu_baseline_batched(p, d, st, args.cpu_seconds) if p.batched
                                else cpu_baseline(p, d, st.ids, st.w, args.cpu_seconds))
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
