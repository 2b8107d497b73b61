"""bench.py's host-side accounting and its one-GPU contract, without a GPU.

The algorithmic counts are restated from the shapes by hand: FLOPs of the
four projections (2 M N K each) and of causal attention (QK^T and PV over the
causal half, 2 B Hl S^2 d), and the decode bytes (the rank's weights once,
K/V of positions 0..L read, one position written).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_flops_70b_t8():
    gemm, attn = bench.prefill_flops(8192, 64, 8, 28672, 8, 4, 4096)
    T = 4 * 4096
    assert gemm["gemm_qkv"] == 2 * T * 8192 * (8 + 2) * 128 == 343597383680
    assert gemm["gemm_out"] == 2 * T * 1024 * 8192 == 274877906944
    assert gemm["gemm_up"] == 2 * T * 8192 * 7168 == 1924145348608
    assert gemm["gemm_down"] == 2 * T * 3584 * 8192 == 962072674304
    assert attn == 2 * 4 * 8 * 4096 * 4096 * 128 == 137438953472
    assert sum(gemm.values()) + attn == 3642132267008


def test_prefill_flops_7b_t2():
    gemm, attn = bench.prefill_flops(4096, 32, 32, 11008, 2, 1, 2048)
    assert gemm["gemm_up"] == 2 * 2048 * 4096 * 11008 == 184683593728
    assert gemm["gemm_qkv"] == 2 * 2048 * 4096 * 48 * 128
    assert attn == 2 * 16 * 2048 * 2048 * 128


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_bytes_70b_t8(fp8):
    total, per = bench.decode_bytes(8192, 64, 8, 28672, 8, 1, 4096, fp8)
    shapes = {"gemv_qkv": (1280, 8192), "gemv_out": (8192, 1024), "gemv_up": (7168, 8192), "gemv_down": (8192, 3584)}
    for k, (n, kk) in shapes.items():
        assert per[k] == (n * kk + 4 * n if fp8 else 2 * n * kk), k
    kv_read = 2 * 2 * 1 * 128 * 4097          # K and V, one KV head, positions 0..4096, bf16
    assert per["attn_decode"] == kv_read
    weights = sum(per[k] for k in shapes)
    assert weights == bench.weight_bytes(8192, 64, 8, 28672, 8, fp8)
    assert total == weights + kv_read + 2 * 2 * 128   # plus the appended position
    if not fp8:
        assert weights == 213909504


def test_decode_bytes_scale_with_batch():
    t1, _ = bench.decode_bytes(4096, 32, 32, 11008, 4, 1, 1024)
    t3, _ = bench.decode_bytes(4096, 32, 32, 11008, 4, 3, 1024)
    kv1 = 2 * 2 * 8 * 128 * (1024 + 1) + 2 * 2 * 8 * 128
    assert t3 - t1 == 2 * kv1                      # weights once, K/V per sequence
