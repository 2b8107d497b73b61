"""Host-side checks of the C ABI (no GPU needed).

- the built library exports every function include/tp_shard.h declares;
- tp_shard_create applies the partition rules (golden cases, with their
  citations in tests/golden/partition_cases.txt) and the kernel limits
  before touching a device;
- argument and state errors of the other entry points return their codes
  without launching anything.
"""

import ctypes as C
import os
import re

import pytest

from tensor_transformer_layer_tp_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "partition_cases.txt")

pytestmark = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="libtpshard.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = N.lib()
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(n for n, _, _ in N.SIGNATURES) == names


def test_status_strings():
    lib = N.lib()
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -99):
        assert lib.tp_status_string(code)


def create(hidden, heads, kv, ffn, t, r, dtype=N.TP_BF16, act=N.TP_ACT_SWIGLU, rope=1):
    opts = N.tp_opts(dtype, act, 1, 1e-5, rope, 10000.0)
    h = C.c_void_p()
    st = N.lib().tp_shard_create(hidden, heads, kv, ffn, t, r, C.byref(opts), C.byref(h))
    if st == N.TP_OK:
        N.lib().tp_shard_destroy(h)
    return st


def golden_cases():
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            H, Hk, Fw, t, e = line.split()
            out.append((int(H), int(Hk), int(Fw), int(t), e))
    return out


@pytest.mark.parametrize("case", golden_cases(), ids=str)
def test_create_partition_rules(case):
    H, Hk, Fw, t, expect = case
    st = create(H * 128, H, Hk, Fw, t, 0)
    if expect == "divide":
        assert st == N.TP_E_DIVIDE
    else:
        # allowed by the pages; the kernels additionally need (ffn/t) % 64 == 0
        assert st == (N.TP_OK if (Fw // t) % 64 == 0 else N.TP_E_ARG)


def test_create_rank_and_args():
    assert create(4096, 32, 32, 11008, 2, 2) == N.TP_E_RANK
    assert create(4096, 32, 32, 11008, 2, -1) == N.TP_E_RANK
    assert create(4096, 32, 32, 11008, 0, 0) == N.TP_E_ARG
    assert create(4000, 32, 32, 11008, 2, 0) == N.TP_E_ARG          # hidden % heads
    assert create(4096, 32, 5, 11008, 1, 0) == N.TP_E_ARG           # heads % kv_heads
    assert create(4096, 16, 16, 11008, 2, 0) == N.TP_E_ARG          # head_dim 256 unsupported
    assert create(256, 4, 4, 1024, 2, 1, dtype=N.TP_F32, act=N.TP_ACT_GELU, rope=0) == N.TP_OK
    assert create(4096, 32, 32, 11008, 2, 1) == N.TP_OK
    assert create(8192, 64, 8, 28672, 8, 7) == N.TP_OK
    assert N.lib().tp_shard_create(64, 1, 1, 64, 1, 0, None, None) == N.TP_E_ARG
    bad = N.tp_opts(7, 0, 1, 1e-5, 1, 1e4)
    h = C.c_void_p()
    assert N.lib().tp_shard_create(4096, 32, 32, 11008, 2, 0, C.byref(bad), C.byref(h)) == N.TP_E_ARG


def test_forward_before_weights_is_state_error():
    lib = N.lib()
    h = C.c_void_p()
    assert lib.tp_shard_create(4096, 32, 32, 11008, 2, 0, None, C.byref(h)) == N.TP_OK
    fake = C.c_void_p(0x10000)  # never dereferenced: validation comes first
    try:
        assert lib.tp_shard_forward_prefill(h, N.TP_STAGE_ATTN, fake, 1, 16, None, fake, None) == N.TP_E_STATE
        assert lib.tp_shard_forward_decode(h, N.TP_STAGE_MLP, fake, 1, None, fake, None) == N.TP_E_STATE
        assert lib.tp_shard_forward_prefill(h, 5, fake, 1, 16, None, fake, None) == N.TP_E_ARG
        assert lib.tp_shard_forward_prefill(h, 0, C.c_void_p(0x10002), 1, 16, None, fake, None) == N.TP_E_ARG
        assert lib.tp_shard_forward_prefill(h, 0, fake, 0, 16, None, fake, None) == N.TP_E_ARG
        assert lib.tp_shard_forward_prefill(h, 0, None, 1, 16, None, fake, None) == N.TP_E_ARG
        assert lib.tp_shard_reserve(h, 0) == N.TP_E_ARG
        p = C.c_void_p()
        assert lib.tp_shard_debug_view(h, 0, C.byref(p)) == N.TP_E_ARG   # no workspace yet
        w = N.tp_weights()
        assert lib.tp_shard_load_weights(h, C.byref(w), None) == N.TP_E_ARG  # NULL weights
    finally:
        lib.tp_shard_destroy(h)


def test_decode_reduce_argument_and_state_errors():
    """tp_shard_forward_decode_reduce validates on the host before any
    device call: missing pointers, a lost other rank, misalignment and an
    output overlapping the input are argument errors; a shard without
    weights is a state error."""
    lib = N.lib()
    h = C.c_void_p()
    assert lib.tp_shard_create(4096, 32, 8, 11008, 2, 1, None, C.byref(h)) == N.TP_OK
    x, out, p0 = 0x100000, 0x200000, 0x300000
    parts = (C.c_void_p * 2)(p0, None)          # rank 1's own slot may be NULL
    f = lib.tp_shard_forward_decode_reduce
    try:
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, parts, None, C.c_void_p(out), None) == N.TP_E_STATE
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, None, None, C.c_void_p(out), None) == N.TP_E_ARG
        lost = (C.c_void_p * 2)(None, p0)       # rank 0's partial missing
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, lost, None, C.c_void_p(out), None) == N.TP_E_ARG
        mis = (C.c_void_p * 2)(p0 + 4, None)
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, mis, None, C.c_void_p(out), None) == N.TP_E_ARG
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, parts, None, C.c_void_p(out + 8), None) == N.TP_E_ARG
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, parts, C.c_void_p(x + 2), C.c_void_p(out),
                 None) == N.TP_E_ARG                                    # misaligned residual
        # out overlapping x (4096 bf16 values = 8 KB per sequence)
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, parts, None, C.c_void_p(x + 4096), None) == N.TP_E_ARG
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 2, None, parts, None, C.c_void_p(x + 8192), None) == N.TP_E_ARG
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 1, None, parts, None, C.c_void_p(x + 8192), None) == N.TP_E_STATE
        assert f(h, N.TP_STAGE_MLP, C.c_void_p(x), 0, None, parts, None, C.c_void_p(out), None) == N.TP_E_ARG
    finally:
        lib.tp_shard_destroy(h)


def test_prefill_reduce_argument_and_state_errors():
    """tp_shard_forward_prefill_reduce validates on the host before any
    device call: missing pointers, a lost other rank, misalignment and an
    output overlapping the input or another rank's partial are argument
    errors; a shard without weights is a state error."""
    lib = N.lib()
    h = C.c_void_p()
    assert lib.tp_shard_create(4096, 32, 8, 11008, 2, 1, None, C.byref(h)) == N.TP_OK
    x, out, p0 = 0x1000000, 0x2000000, 0x3000000   # 16 tokens of 4096 bf16 = 128 KB, fp32 partials 256 KB
    parts = (C.c_void_p * 2)(p0, None)              # rank 1's own slot may be NULL
    f = lib.tp_shard_forward_prefill_reduce
    M = N.TP_STAGE_MLP
    try:
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(out), None) == N.TP_E_STATE
        assert f(h, M, C.c_void_p(x), 1, 16, None, None, None, C.c_void_p(out), None) == N.TP_E_ARG
        lost = (C.c_void_p * 2)(None, p0)           # rank 0's partial missing
        assert f(h, M, C.c_void_p(x), 1, 16, None, lost, None, C.c_void_p(out), None) == N.TP_E_ARG
        mis = (C.c_void_p * 2)(p0 + 4, None)
        assert f(h, M, C.c_void_p(x), 1, 16, None, mis, None, C.c_void_p(out), None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(out + 8), None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, C.c_void_p(x + 2), C.c_void_p(out), None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, None, None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 0, None, parts, None, C.c_void_p(out), None) == N.TP_E_ARG
        # out overlapping x (16 x 4096 bf16 = 128 KB) or rank 0's partial (256 KB)
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(x + 65536), None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(p0 + 196608), None) == N.TP_E_ARG
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(p0 + 262144), None) == N.TP_E_STATE
        assert f(h, M, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(x + 131072), None) == N.TP_E_STATE
        assert f(h, 7, C.c_void_p(x), 1, 16, None, parts, None, C.c_void_p(out), None) == N.TP_E_ARG
    finally:
        lib.tp_shard_destroy(h)


def test_partial_reduce_argument_errors():
    lib = N.lib()
    fake = 0x10000
    out = C.c_void_p(0x20000)
    arr = (C.c_void_p * 2)(fake, fake)
    assert lib.tp_partial_reduce(arr, 0, None, out, 16, N.TP_BF16, None) == N.TP_E_ARG
    assert lib.tp_partial_reduce(arr, 65, None, out, 16, N.TP_BF16, None) == N.TP_E_ARG
    lost = (C.c_void_p * 2)(fake, None)                           # a lost rank
    assert lib.tp_partial_reduce(lost, 2, None, out, 16, N.TP_BF16, None) == N.TP_E_ARG
    mis = (C.c_void_p * 2)(fake, fake + 4)
    assert lib.tp_partial_reduce(mis, 2, None, out, 16, N.TP_BF16, None) == N.TP_E_ARG
    assert lib.tp_partial_reduce(arr, 2, None, None, 16, N.TP_BF16, None) == N.TP_E_ARG
    assert lib.tp_partial_reduce(arr, 2, None, out, 16, 9, None) == N.TP_E_ARG
    assert lib.tp_partial_reduce(arr, 2, None, out, 0, N.TP_BF16, None) == N.TP_OK   # nothing to do


def test_kv_argument_errors():
    lib = N.lib()
    n = C.c_int()
    assert lib.tp_kv_set_len(None, 3) == N.TP_E_ARG
    assert lib.tp_kv_get_len(None, C.byref(n)) == N.TP_E_ARG
    assert lib.tp_kv_view(None, None, None) == N.TP_E_ARG
    assert lib.tp_kv_create(None, 1, 16, C.byref(C.c_void_p())) == N.TP_E_ARG
    assert lib.tp_kv_set_len_async(None, 3, None) == N.TP_E_ARG
    assert lib.tp_kv_get_len_stream(None, C.byref(n), None) == N.TP_E_ARG


def test_tune_hook_range():
    lib = N.lib()
    assert lib.tp_tune_set_gemm_config(99) == N.TP_E_ARG
    assert lib.tp_tune_set_gemm_config(-1) == N.TP_OK
    assert lib.tp_tune_set_attn_groups(3) == N.TP_E_ARG
    assert lib.tp_tune_set_attn_groups(-1) == N.TP_E_ARG
    assert lib.tp_tune_set_attn_groups(0) == N.TP_OK
    assert lib.tp_tune_set_attn_kernel(3) == N.TP_E_ARG
    assert lib.tp_tune_set_attn_kernel(-1) == N.TP_E_ARG
    assert lib.tp_tune_set_attn_kernel(0) == N.TP_OK
    assert lib.tp_tune_set_decode_chunk(48) == N.TP_E_ARG
    assert lib.tp_tune_set_decode_chunk(0) == N.TP_OK


def test_fp8_option_rules():
    """decode_fp8 needs the bf16 shard; the fp8 view needs loaded weights."""
    lib = N.lib()
    h = C.c_void_p()
    bad = N.tp_opts(N.TP_F32, N.TP_ACT_SWIGLU, 1, 1e-5, 1, 10000.0, 1)
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, C.byref(bad), C.byref(h)) == N.TP_E_ARG
    bad2 = N.tp_opts(N.TP_BF16, N.TP_ACT_SWIGLU, 1, 1e-5, 1, 10000.0, 2)
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, C.byref(bad2), C.byref(h)) == N.TP_E_ARG
    ok = N.tp_opts(N.TP_BF16, N.TP_ACT_SWIGLU, 1, 1e-5, 1, 10000.0, 1)
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, C.byref(ok), C.byref(h)) == N.TP_OK
    q, sc, r, c = C.c_void_p(), C.c_void_p(), C.c_int(), C.c_int()
    assert lib.tp_shard_fp8_view(h, 0, C.byref(q), C.byref(sc), C.byref(r), C.byref(c)) == N.TP_E_STATE
    assert lib.tp_shard_fp8_view(h, 4, C.byref(q), C.byref(sc), C.byref(r), C.byref(c)) == N.TP_E_ARG
    lib.tp_shard_destroy(h)


def test_sequence_parallel_argument_rules():
    """Argument checks of the reduce-scatter, all-gather and norm entry points
    (all detected on the host before any device work)."""
    lib = N.lib()
    fake = C.c_void_p(1 << 20)            # 16-byte aligned, never dereferenced
    parts = (C.c_void_p * 2)(fake, fake)
    rs = lib.tp_partial_reduce_scatter
    assert rs(parts, 2, 0, None, fake, 11, 64, N.TP_BF16, None) == N.TP_E_DIVIDE    # rows % t
    assert rs(parts, 2, 0, None, fake, 10, 60, N.TP_BF16, None) == N.TP_E_ARG       # cols % 8
    assert rs(parts, 2, 2, None, fake, 10, 64, N.TP_BF16, None) == N.TP_E_RANK      # rank >= t
    assert rs(parts, 2, 0, None, fake, 10, 64, 7, None) == N.TP_E_ARG               # dtype
    assert rs(parts, 2, 0, None, fake, 0, 64, N.TP_BF16, None) == N.TP_OK           # nothing to do
    ag = lib.tp_all_gather
    assert ag(parts, 2, 4, 4, N.TP_BF16, fake, None) == N.TP_E_ARG                  # 8-byte rows
    assert ag(parts, 2, 0, 64, N.TP_BF16, fake, None) == N.TP_OK
    assert ag(parts, 0, 4, 64, N.TP_BF16, fake, None) == N.TP_E_ARG
    h = C.c_void_p()
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, None, C.byref(h)) == N.TP_OK
    assert lib.tp_shard_norm(h, 3, fake, 4, fake, None) == N.TP_E_ARG
    assert lib.tp_shard_norm(h, 1, fake, 4, fake, None) == N.TP_E_STATE             # no weights yet
    lib.tp_shard_destroy(h)


def test_paged_cache_argument_rules():
    """Paged caches need a bf16 shard and a power-of-two block size in [16, 1024]."""
    lib = N.lib()
    h, kv = C.c_void_p(), C.c_void_p()
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, None, C.byref(h)) == N.TP_OK
    for bs in (0, 8, 24, 2048):
        assert lib.tp_kv_create_paged(h, 1, 64, bs, 16, C.byref(kv)) == N.TP_E_ARG
    assert lib.tp_kv_create_paged(h, 1, 64, 16, 0, C.byref(kv)) == N.TP_E_ARG
    assert lib.tp_kv_set_block_table(None, None) == N.TP_E_ARG
    lib.tp_shard_destroy(h)
    f32 = N.tp_opts(N.TP_F32, N.TP_ACT_SWIGLU, 1, 1e-5, 1, 10000.0, 0)
    assert lib.tp_shard_create(512, 8, 8, 1024, 2, 0, C.byref(f32), C.byref(h)) == N.TP_OK
    assert lib.tp_kv_create_paged(h, 1, 64, 16, 16, C.byref(kv)) == N.TP_E_ARG
    lib.tp_shard_destroy(h)


def test_gemm_plan_column_splits():
    """The planner's launch plans (host only): the shapes for which it runs
    a projection as two launches over column ranges, the forced split hook,
    and that every plan covers all N columns with 64-aligned split points."""
    from tensor_transformer_layer_tp_amd import gemm_plan, set_gemm_split
    lib = N.lib()
    # unsharded 7B gate/up at 2048 tokens (crossover sweep B1 S2048, B4 S512, B16 S128)
    assert [c for _, c in gemm_plan(2048, 22016, 4096, "swiglu")] == [16384, 5632]
    # sharded 7B gate/up at 8192 tokens (B1 S8192, B4 S2048, B16 S512, B64 S128)
    assert [c for _, c in gemm_plan(8192, 11008, 4096, "swiglu")] == [10240, 768]
    # 70B t=8 Q/K/V projection (B4 S4096)
    assert len(gemm_plan(16384, 1280, 8192, "qkv")) == 2
    # the 7B t=2 prefill at 2048 tokens: single launches, gate/up on the four-wave 256x192 tile
    assert gemm_plan(2048, 11008, 4096, "swiglu") == [(17, 11008)]
    assert len(gemm_plan(2048, 6144, 4096, "qkv")) == 1
    for M in (1, 128, 300, 2048, 8192, 16384, 524288):
        for N_, K, kind in ((6144, 4096, "qkv"), (12288, 4096, "qkv"), (1280, 8192, "qkv"), (11008, 4096, "swiglu"),
                            (22016, 4096, "swiglu"), (7168, 8192, "swiglu"), (4096, 5504, "partial"),
                            (8192, 1024, "partial"), (1408, 1024, "gelu")):
            plan = gemm_plan(M, N_, K, kind)
            assert sum(c for _, c in plan) == N_
            assert all(c % 64 == 0 for _, c in plan[:-1])
            assert all(0 <= cfg < 19 for cfg, _ in plan)
            if kind == "qkv":   # the four-wave 256x192 tile has no room for the rotary epilogue
                assert all(cfg != 17 for cfg, _ in plan)
    try:
        set_gemm_split(14, 16, 640)
        assert gemm_plan(2048, 11008, 4096, "swiglu") == [(14, 640), (16, 10368)]
        assert len(gemm_plan(300, 512, 1024, "qkv")) == 1   # not wider than the split: the planner's plan
    finally:
        set_gemm_split(0, 0, 0)
    assert len(gemm_plan(2048, 11008, 4096, "swiglu")) == 1
    assert lib.tp_tune_set_gemm_split(14, 16, 100) == N.TP_E_ARG      # not a multiple of 64
    assert lib.tp_tune_set_gemm_split(99, 16, 640) == N.TP_E_ARG      # no such configuration
    assert lib.tp_tune_set_gemm_split(14, 16, -64) == N.TP_E_ARG
    parts, cfg, cols = C.c_int(), (C.c_int * 2)(), (C.c_int * 2)()
    assert lib.tp_tune_gemm_plan(0, 64, 64, N.TP_PROJ_QKV, C.byref(parts), cfg, cols) == N.TP_E_ARG
    assert lib.tp_tune_gemm_plan(64, 64, 64, 7, C.byref(parts), cfg, cols) == N.TP_E_ARG
