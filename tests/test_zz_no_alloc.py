"""The allocation-free decode entry point, tp_shard_forward_decode_noalloc,
called through the C ABI and compared with the allocating entry point
tp_shard_forward_decode on twin shards (same weights, same caches): two
calls in a row, the second with a smaller input, each an ATTN stage
(appending to the cache) and an MLP stage.  The outputs and the appended
cache rows must be identical (the same kernels on the same values) and
match the oracle; the device's free memory must not move across the
allocation-free calls; a call whose workspace exceeds the static array is
refused before any launch."""

from __future__ import annotations

import ctypes as C

import numpy as np
import pytest
import torch

from oracle import layer as O
from tensor_transformer_layer_tp_amd import ATTN, MLP, _native as N, synth

from helpers import Layer, assert_close, to_np

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


def ptr(t):
    return C.c_void_p(t.data_ptr())


def decode(fn, sh, stage, x, kv, out):
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(sh._h, stage, ptr(x), int(x.shape[0]), kv._h if kv is not None else None, ptr(out), st)


def test_noalloc_decode_matches_allocating_entry_point():
    lib = N.lib()
    hid, t, r = 1024, 2, 1
    L = Layer(hid, 8, 4, 2816, batch=3, seq=44, gamma_noise=True, seed=91)
    sh_a, sh_n = L.shard(t, r), L.shard(t, r)
    # first call: 3 sequences (split-K projections), cache capacity 300;
    # second call: 1 sequence (GEMV projections), capacity 64
    for call, (B, S, cap) in enumerate(((3, 40, 300), (1, 20, 64))):
        announce(f"allocation-free decode, call {call + 1}: batch {B}, prompt {S}, cache capacity {cap}")
        x_pre = L.dev["x"][:B, :S].contiguous()
        kv_a, kv_n = sh_a.kv_cache(B, cap), sh_n.kv_cache(B, cap)
        sh_a.prefill(ATTN, x_pre, kv_a)
        sh_n.prefill(ATTN, x_pre, kv_n)
        xd = L.dev["x"][:B, S].contiguous()
        h = synth.to_storage(synth.draw_normal((B, hid), 92 + call), "bf16").cuda()
        pa_a = torch.full((B, hid), float("nan"), device="cuda")
        pm_a = torch.full_like(pa_a, float("nan"))
        pa_n = torch.full_like(pa_a, float("nan"))
        pm_n = torch.full_like(pa_a, float("nan"))
        assert decode(lib.tp_shard_forward_decode, sh_a, ATTN, xd, kv_a, pa_a) == N.TP_OK
        assert decode(lib.tp_shard_forward_decode, sh_a, MLP, h, None, pm_a) == N.TP_OK
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        assert decode(lib.tp_shard_forward_decode_noalloc, sh_n, ATTN, xd, kv_n, pa_n) == N.TP_OK
        assert decode(lib.tp_shard_forward_decode_noalloc, sh_n, MLP, h, None, pm_n) == N.TP_OK
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0, "device memory changed across the allocation-free calls"
        assert torch.equal(pa_n, pa_a), f"call {call + 1}: attention partial differs from the allocating call"
        assert torch.equal(pm_n, pm_a), f"call {call + 1}: MLP partial differs from the allocating call"
        assert kv_n.length == S + 1
        ka, va = kv_a.read()
        kn, vn = kv_n.read()
        torch.cuda.synchronize()
        assert torch.equal(ka, kn) and torch.equal(va, vn)
        # and the oracle
        pre = O.attn_stage(L.exact["x"][:B, :S], L.W, L.spec, t, r)
        ref = O.decode_attn_stage(L.exact["x"][:B, S], pre["k"], pre["v"], L.W, L.spec, t, r)
        assert_close(to_np(pa_n), ref["partial"], f"call {call + 1}: attention partial vs oracle", "bf16")
        assert_close(to_np(kn)[:, :, S], ref["k_new"], f"call {call + 1}: appended k vs oracle", "bf16")
        refm = O.mlp_stage(h.float().cpu().numpy()[:, None], L.W, L.spec, t, r)
        assert_close(to_np(pm_n), refm["partial"][:, 0], f"call {call + 1}: MLP partial vs oracle", "bf16")
        kv_a.close()
        kv_n.close()
    # a workspace beyond the static array: refused before any launch
    announce("allocation-free decode beyond the static array")
    B, cap = 8, 200000
    kv_big = sh_n.kv_cache(B, cap)
    xb = torch.zeros((B, hid), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, hid), 5.0, device="cuda")
    assert decode(lib.tp_shard_forward_decode_noalloc, sh_n, ATTN, xb, kv_big, out) == N.TP_E_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(out == 5.0)) and kv_big.length == 0
    kv_big.close()
