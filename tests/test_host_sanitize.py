"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tsp_api.cpp (validation, planner, workspace carving, launch composition) and
layout.cpp (the kernels' host-side sizes) are compiled with g++ and the two
sanitizers, without any device code: the kernel launches are replaced by the
recording stand-ins of tests/host_check/stubs.cpp, which check each launch's
preconditions and that every byte range its kernel would touch lies inside a
caller buffer.  tests/host_check/host_check.cpp calls every public entry point
on buffers sized exactly as include/tsp.h documents them (shapes with D = 1 and
TSP_MAX_D, ragged chunks, head_dim 64 and 128, split and unsplit attention
grids, grouped-query heads, zero tokens) and every rejection path (status
returned, nothing launched).  Needs g++ only; no GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "host_check")
CSRC = os.path.join(ROOT, "folded_tensor_sequence_tsp_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


def test_host_layer_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", HC, os.path.join(CSRC, "tsp_api.cpp"), os.path.join(CSRC, "layout.cpp"),
           os.path.join(HC, "stubs.cpp"), os.path.join(HC, "host_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"host check failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "kernel launches checked" in r.stdout
