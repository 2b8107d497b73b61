"""The host runtime (tp_shard.cpp) under AddressSanitizer and UBSan, on the CPU.

tests/host_sanitizer/ holds host test doubles for the HIP runtime calls and
the kernel launchers that the runtime makes -- device memory becomes host
memory in a registry, and every launcher checks that each range its kernel
would read or write lies inside one live allocation -- and a driver that
walks the whole C ABI: the partition and argument errors, calls out of order
(a forward pass before the weights, a decode MLP stage before any ATTN
stage), every prefill and decode path of bf16, fp32, GELU, E4M3 and paged
shards, the reduce calls, the allocation-free entry point, the timer, and a
failure injected into each device allocation the weight loader, the
workspace and the caches make (including the second of an E4M3 code/scale
pair), each followed by a retry and a leak check.  The GPU kernels
themselves are not compiled into this sanitized executable (the parity
tests cover them); only the host code is instrumented.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = [
    os.path.join(ROOT, "tensor_transformer_layer_tp_amd", "csrc", "tp_shard.cpp"),
    os.path.join(ROOT, "tests", "host_sanitizer", "hip_doubles.cpp"),
    os.path.join(ROOT, "tests", "host_sanitizer", "driver.cpp"),
]


def _build(tmp_path):
    if not os.path.exists(CLANG) or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("ROCm clang++ and HIP headers are needed for the host build")
    exe = str(tmp_path / "host_driver")
    cmd = [CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-DHIP_SYMBOL(X)=X", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")] + SOURCES + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_host_runtime_under_sanitizers(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "0 failed" in r.stdout, out[-2000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
