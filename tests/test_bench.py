"""bench.py's host logic on the CPU: the one-GPU contract, the algorithmic FLOP and
byte counts behind `value` and the rooflines, and the traffic lookup that only
trusts a profile taken on the current kernel sources."""
import importlib.util
import json
import os
import re
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = load_bench()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["gpus_requested"] == 2


def test_algorithmic_counts_bf16_and_fp8():
    p = synth.Problem(M=10, H=256, I=384, E=6, topk=2, block_m=16)
    a = bench.algorithmic(p, touched=5)
    R = p.M * p.topk
    assert a["flops"] == 6.0 * R * p.H * p.I and a["flops_g1"] == 4.0 * R * p.H * p.I
    w = 5 * 3 * p.I * p.H * 2                       # touched experts' w13 and w2, bf16
    assert a["bytes"] == w + 2 * p.M * p.H * 2 + p.M * p.E * 4
    # GEMM1 reads w13 and x, writes h (2I columns) or, fused, z (I columns)
    assert a["bytes_g1"] == 5 * 2 * p.I * p.H * 2 + p.M * p.H * 2 + R * 2 * p.I * 2
    assert bench.algorithmic(p, 5, act_fused=True)["bytes_g1"] == a["bytes_g1"] - R * p.I * 2
    q = synth.Problem(M=10, H=256, I=384, E=6, topk=2, block_m=128, wdtype="fp8")
    b = bench.algorithmic(q, touched=5)
    assert b["flops"] == a["flops"]
    wq = 5 * 3 * q.I * q.H * (1 + 4.0 / (128 * 128))  # e4m3 + fp32 block scales
    assert abs(b["bytes"] - (wq + 2 * q.M * q.H * 2 + q.M * q.E * 4)) < 1e-6


def test_stage_work_adds_up_to_the_layer():
    p = synth.Problem(M=64, H=512, I=256, E=8, topk=2, block_m=16)
    R, npp = 128, 192
    w = bench.stage_work(p, touched=8, R=R, npp=npp, act_fused=True)
    assert set(w) == {"router", "align", "gemm1", "gemm2", "reduce"}
    assert w["gemm1"]["flops"] + w["gemm2"]["flops"] == 6.0 * R * p.H * p.I
    unfused = bench.stage_work(p, 8, R, npp, act_fused=False)
    # without the fusion GEMM1 writes h and a separate pass turns it into z
    assert unfused["act"]["bytes"] == npp * 2 * p.I * 2 + npp * p.I * 2
    q = synth.Problem(M=64, H=512, I=256, E=8, topk=2, block_m=128, wdtype="fp8")
    assert "quant" in bench.stage_work(q, 8, R, npp, True)


def test_stage_roofline_classification():
    work = {"tiny": {"bytes": 1000}, "stream": {"bytes": 8e9}, "gemm": {"bytes": 1e6, "flops": 2.5e12}}
    r = bench.stage_roofline(work, {"tiny": 0.005, "stream": 2.0, "gemm": 2.0}, "bf16")
    assert r["tiny"]["bound"] == "latency" and r["tiny"]["us"] == 5.0
    assert r["stream"]["bound"] == "hbm" and abs(r["stream"]["frac"] - 0.5) < 1e-9
    assert r["stream"]["achieved"] == 4000.0
    assert r["gemm"]["bound"] == "mfma" and abs(r["gemm"]["frac"] - 0.5) < 1e-9


K128 = "kernel = void expert_gemm_dma_kernel<dma::Cfg<128, 512, 1, 4, 64, 8>, true, true>(GemmArgs)\n"


def test_traffic_needs_a_profile_of_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("w", 128) is None                 # no profile
    f = tmp_path / "gemm1_w_traffic.txt"
    f.write_text("# header\n" + K128 + "hbm_bytes_per_launch = 1234\nkernel_source_sha256 = 0\n")
    assert bench.measured_traffic("w", 128) is None                 # other sources
    f.write_text(K128 + f"hbm_bytes_per_launch = 1234\nkernel_source_sha256 = {bench.kernel_source_digest()}\n")
    assert bench.measured_traffic("w", 128) == 1234.0
    assert bench.measured_traffic("w", 256) is None                 # taken with another block_m


def test_mfma_counters_need_a_profile_of_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_mfma("w", 128) is None
    f = tmp_path / "gemm1_w_mfma.txt"
    body = K128 + "mfma_busy_fraction = 0.5   (note)\nclock_ghz = 1.8   (note)\n"
    f.write_text(body + "kernel_source_sha256 = 0\n")
    assert bench.measured_mfma("w", 128) is None
    f.write_text(body + f"kernel_source_sha256 = {bench.kernel_source_digest()}\n")
    assert bench.measured_mfma("w", 128) == {"busy_fraction": 0.5, "clock_ghz": 1.8}
    assert bench.measured_mfma("w", 256) is None


def test_profile_block_m_from_the_kernel_name():
    assert bench.profile_block_m(K128.split("=", 1)[1]) == 128
    assert bench.profile_block_m("expert_gemm_dma_kernel<dma::Cfg<256, 256, 2, 5, 64, 8>, true, true>") == 256
    assert bench.profile_block_m("expert_gemm_fp8_kernel<f8::Cfg<128, 256, 2, 4, 3, false>, true, true, 0>") == 128
    assert bench.profile_block_m("stream_gemm_bf16_kernel<true, true, 2, 4, 4, true, true>") == 16
    assert bench.profile_block_m("something else") == -1


def test_committed_profiles_name_the_sources_they_were_taken_on():
    # every GEMM1 counter profile under profiles/ records the digest of the kernel
    # sources it was measured on; bench.py reports its figures only while the sources
    # still hash to that value (see the two tests above), and null after a change
    files = [n for n in os.listdir(os.path.join(ROOT, "profiles"))
             if n.endswith("_traffic.txt") or n.endswith("_mfma.txt")]
    assert files
    for n in files:
        text = open(os.path.join(ROOT, "profiles", n)).read()
        assert re.search(r"^kernel_source_sha256 = [0-9a-f]{64}$", text, re.M), n


def test_cpu_model_names_the_host():
    # the model name, its family / model numbers where /proc/cpuinfo has them, and
    # the logical CPU count
    s = bench.cpu_model()
    assert s == "unknown" or s.endswith("logical CPUs)")
    if os.path.exists("/proc/cpuinfo") and "cpu family" in open("/proc/cpuinfo").read():
        assert "cpu family" in s
