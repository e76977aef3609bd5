"""Host logic of the C ABI under the address and undefined-behaviour sanitizers (CPU).

``tests/host/host_abi_test.cpp`` drives ``vlca_api.cpp`` compiled with g++
against a stand-in HIP runtime (``tests/host/hip_stub.cpp``): argument errors,
the launch plan and split settings, and the per-stream worklist and split-pool
bookkeeping (no stream synchronisation, nothing freed that a captured graph may
still use, state created during a capture without recording into it), the
no-allocation entry point's scratch layout, and the bucketed graph runner
(bucket choice, pre-capture and lazy capture, device-side offset padding,
eager fallback).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SOURCES = [os.path.join(HOST, "host_abi_test.cpp"), os.path.join(HOST, "hip_stub.cpp"),
           os.path.join(ROOT, "varlen_causal_attention_amd", "csrc", "vlca_api.cpp"),
           os.path.join(ROOT, "varlen_causal_attention_amd", "csrc", "vlca_graph.cpp")]


def test_host_abi_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "host_abi_test")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "varlen_causal_attention_amd", "csrc"),
           *SOURCES, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    # The library keeps every worklist and pool until the process ends (a captured
    # graph may still use them), so leak detection is off; use-after-free is not.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and "ALL OK" in run.stdout, run.stdout + run.stderr
