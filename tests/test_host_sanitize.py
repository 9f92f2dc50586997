"""The plan's host code (descriptor validation, Hilbert ranks, block and
sub-block tables) under AddressSanitizer and UndefinedBehaviorSanitizer: a
sweep of valid and invalid descriptors through fva_plan_dims and
fva_plan_tables, built with the host compiler (no GPU code involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                    reason="needs g++ and the HIP runtime library")
def test_plan_host_code_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_sanitize"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{ROOT}/block_sparse_spatiotemporal_amd/csrc",
           f"{ROOT}/tests/host/plan_sanitize.cpp", f"{ROOT}/block_sparse_spatiotemporal_amd/csrc/plan.cpp",
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip().startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
