"""The oracle and the library's host-side code under AddressSanitizer and UBSan (CPU only).

* The oracle is rebuilt with gcc -fsanitize=address,undefined and the oracle's
  pin tests run against that build (MOE_ORACLE_SO), the sanitizer runtimes
  preloaded into the test process. Any out-of-bounds access, use after free or
  undefined behaviour aborts the run.
* libmoe.so is rebuilt with the same sanitizers on its host code only (the GPU
  code is built as usual) and the C ABI tests, which reach every validation
  path and status code, run against it (MOE_LIB_PATH).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))) + [
    os.path.join(ROOT, "tests", "test_sampled.py")]


def run_pytest(files, env_extra, timeout):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    so = str(tmp_path / "libmoe_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", so, os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"],
                   check=True)
    rt = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                                 check=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    run_pytest(ORACLE_TESTS, {"MOE_ORACLE_SO": so, "LD_PRELOAD": rt, "OMP_NUM_THREADS": "4"}, 1200)


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("no clang ASan runtime in this image")
    so = str(tmp_path / "libmoe_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_ffn_block_amd", "csrc", "*.hip")))
    # the sanitizer flags reach the host compilation only
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-o", so, *srcs]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    run_pytest([os.path.join(ROOT, "tests", "test_abi.py")], {"MOE_LIB_PATH": so, "LD_PRELOAD": rts[0]}, 600)
