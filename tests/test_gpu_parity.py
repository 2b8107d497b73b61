"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name before touching the GPU.  Sizes span several
GEMM and attention tiles with ragged tails; the full-size layers are checked
in full where the oracle finishes in seconds and on sampled rows otherwise.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import layer as O
from tensor_transformer_layer_tp_amd import (ATTN, MLP, PRENORM, Shard, TPError, TP_E_KV_FULL, all_gather,
                                             partial_reduce, partial_reduce_scatter, synth)

from helpers import Layer, assert_close, rank_cache, sum_magnitude, to_np

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


def nan_like(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def run_chain(layer: Layer, tp: int, B: int, S: int, check_kv=True):
    """All tp ranks of a prefill: ATTN stages, reduce, MLP stages, reduce.

    Every stage is compared with the oracle on identical inputs: the ATTN
    stages on x, the reduce on the ranks' partials, the MLP stages on the
    oracle's h (bf16 values, so exactly representable as GPU input).  The
    fully chained GPU result (MLP on the GPU's own h) carries the in-tolerance
    difference between the two h's through the FFN, so it is compared
    norm-wise (relative Frobenius error <= 1e-2)."""
    dt = layer.dtype
    x_dev = layer.dev["x"]
    hid = layer.spec.hidden
    ref = O.layer(layer.exact["x"], layer.W, layer.spec, t=tp)
    shards = [layer.shard(tp, r) for r in range(tp)]
    kvs = [sh.kv_cache(B, S + 5) for sh in shards]
    pa = [sh.prefill(ATTN, x_dev, kv, out=nan_like((B, S, hid))) for sh, kv in zip(shards, kvs)]
    torch.cuda.synchronize()
    for r in range(tp):
        assert_close(to_np(pa[r]), ref["attn"][r]["partial"], f"attn partial r{r}", dt)
        if check_kv:
            k, v = kvs[r].read()
            assert_close(to_np(k)[:, :, :S], ref["attn"][r]["k"], f"K cache r{r}", dt)
            assert_close(to_np(v)[:, :, :S], ref["attn"][r]["v"], f"V cache r{r}", dt)
            assert kvs[r].length == S
    h = partial_reduce(pa, residual=x_dev)
    torch.cuda.synchronize()
    assert_close(to_np(h), ref["h"], "h", dt,
                 sum_magnitude(layer.exact["x"], [a["partial"] for a in ref["attn"]]))
    # MLP stages on the oracle's h
    h_ref = torch.from_numpy(ref["h"].astype(np.float32)).to(layer.torch_dtype).cuda()
    pm = [sh.prefill(MLP, h_ref, out=nan_like((B, S, hid))) for sh in shards]
    y = partial_reduce(pm, residual=h_ref)
    torch.cuda.synchronize()
    for r in range(tp):
        assert_close(to_np(pm[r]), ref["mlp"][r]["partial"], f"mlp partial r{r}", dt)
    assert_close(to_np(y), ref["y"], "y", dt, sum_magnitude(ref["h"], [m["partial"] for m in ref["mlp"]]))
    # fully chained on the GPU's own h
    pm2 = [sh.prefill(MLP, h, out=nan_like((B, S, hid))) for sh in shards]
    y2 = to_np(partial_reduce(pm2, residual=h))
    torch.cuda.synchronize()
    assert np.isfinite(y2).all()
    rel = np.linalg.norm(y2 - ref["y"]) / np.linalg.norm(ref["y"])
    assert rel <= 1e-2, f"chained y: relative Frobenius error {rel:.3g}"
    return shards, kvs


# ---------------------------------------------------------------- reduce kernel

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("t,n", [(1, 1), (2, 3), (3, 4099), (8, 1 << 20), (4, 0), (1, 64), (2, 4096), (4, 4101),
                                 (2, 1 << 22)])
def test_partial_reduce(dtype, t, n):
    announce(f"partial_reduce dtype={dtype} t={t} n={n}")
    parts64 = [synth.draw_normal((n,), 10 + r, 3.0).astype(np.float64) for r in range(t)]
    res = synth.to_storage(synth.draw_normal((n,), 99), dtype)
    parts = [torch.from_numpy(p.astype(np.float32)).cuda() for p in parts64]
    spec = O.Spec(64, 1, 1, 64, mirror_bf16=(dtype == "bf16"))
    if n == 0:
        out = partial_reduce(parts, residual=res.cuda())
        assert out.numel() == 0
        return
    out = partial_reduce(parts, residual=res.cuda())
    p32 = [p.astype(np.float32) for p in parts64]
    want = O.reduce(p32, res.float().numpy(), spec)
    assert_close(to_np(out), want, "reduce", dtype, sum_magnitude(res.float().numpy(), p32))
    out2 = partial_reduce(parts, residual=None, dtype=dtype)
    want2 = O.reduce([p.astype(np.float32) for p in parts64], np.zeros(n), spec)
    assert_close(to_np(out2), want2, "reduce no residual", dtype)


# ---------------------------------------------------------------- whole layers, small

def test_tiny_f32_layer_two_ranks():
    """hidden 256, 4 heads x 64, GELU FFN 1024, fp32, t=2, B=1, S=32, causal."""
    announce("tiny fp32 layer t=2")
    w = synth.WORKLOADS["tiny-f32-t2"]
    L = Layer(w.hidden, w.heads, w.kv_heads, w.ffn, dtype="f32", swiglu=False, norm=False, rope=False,
              batch=1, seq=32)
    run_chain(L, 2, 1, 32)


def test_f32_layer_with_norm_rope_gqa():
    announce("fp32 layer with RMSNorm, RoPE, GQA, t=2, B=2, S=70")
    L = Layer(512, 8, 4, 1024, dtype="f32", batch=2, seq=70, gamma_noise=True, seed=3)
    run_chain(L, 2, 2, 70)


def test_bf16_layer_ragged_gqa_two_ranks():
    announce("bf16 layer hidden 1024, 8 heads, 4 kv heads, ffn 2816, t=2, B=2, S=300")
    L = Layer(1024, 8, 4, 2816, batch=2, seq=300, gamma_noise=True, seed=1)
    shards, _ = run_chain(L, 2, 2, 300)
    # workspace views of the last calls: act of rank 1 on the GPU h is not the
    # oracle's exact input, so only the attention output is compared here
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, 2, 1)
    shards[1].prefill(ATTN, L.dev["x"])
    o = shards[1].debug_tensor("o", (2 * 300, 4 * 128))
    torch.cuda.synchronize()
    assert_close(to_np(o), ref["o"].transpose(0, 2, 1, 3).reshape(600, 512), "attention output o", "bf16")


@pytest.mark.parametrize("kg", [1, 2])
@pytest.mark.parametrize("hidden,heads,kv,S", [(1024, 8, 4, 300), (512, 8, 2, 130)])
def test_attention_key_groups(kg, hidden, heads, kv, S):
    """Prefill attention with one group of waves over every key block and
    with two groups over alternate key blocks whose softmax states merge,
    forced in turn (head dims 128 and 64, GQA, ragged S), against the
    oracle's attention output."""
    from tensor_transformer_layer_tp_amd import set_attn_groups
    announce(f"attention key groups kg={kg} hidden={hidden} heads={heads}/{kv} S={S}")
    t, r, B = 2, 1, 2
    L = Layer(hidden, heads, kv, 2 * hidden, batch=B, seq=S, gamma_noise=True, seed=21)
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, t, r)
    sh = L.shard(t, r)
    hl, d = heads // t, hidden // heads
    try:
        set_attn_groups(kg)
        sh.prefill(ATTN, L.dev["x"])
        o = sh.debug_tensor("o", (B * S, hl * d))
        torch.cuda.synchronize()
    finally:
        set_attn_groups(0)
    assert_close(to_np(o), ref["o"].transpose(0, 2, 1, 3).reshape(B * S, hl * d), f"attention o kg={kg}", "bf16")


def test_bf16_head_dim_64_unsharded():
    announce("bf16 layer head_dim 64, t=1, B=1, S=130")
    L = Layer(512, 8, 2, 1024, batch=1, seq=130, gamma_noise=True, seed=2)
    run_chain(L, 1, 1, 130)


@pytest.mark.parametrize("S", [1, 64, 129])
def test_bf16_sequence_edges(S):
    announce(f"bf16 layer sequence edge S={S}")
    L = Layer(512, 4, 4, 768, batch=1, seq=S, seed=4)
    run_chain(L, 2, 1, S)


def test_bf16_gelu_ffn():
    announce("bf16 layer with GELU FFN, no rope, t=2")
    L = Layer(512, 4, 2, 1024, swiglu=False, rope=False, batch=1, seq=100, seed=5)
    run_chain(L, 2, 1, 100)


def test_bf16_mlp_stage_on_given_h():
    """MLP stage alone on a synthetic h (the oracle's exact input)."""
    announce("bf16 MLP stage on synthetic h, t=4 rank 3")
    L = Layer(1024, 8, 8, 4096, batch=1, seq=0, seed=6, gamma_noise=True)
    h = synth.to_storage(synth.draw_normal((3, 77, 1024), 7), "bf16")
    sh = L.shard(4, 3)
    p = sh.prefill(MLP, h.cuda(), out=nan_like((3, 77, 1024)))
    act = sh.debug_tensor("act", (3 * 77, 1024))
    torch.cuda.synchronize()
    ref = O.mlp_stage(h.float().numpy(), L.W, L.spec, 4, 3)
    assert_close(to_np(act), ref["act"].reshape(3 * 77, 1024), "act", "bf16")
    assert_close(to_np(p), ref["partial"], "mlp partial", "bf16")


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("B", [1, 3, 5, 12])
def test_decode_steps_match_oracle(B):
    announce(f"bf16 decode B={B}: prefill 40 tokens then 3 decode steps, t=2 rank 1")
    S, steps = 40, 3
    L = Layer(1024, 8, 4, 2816, batch=B, seq=S + steps, gamma_noise=True, seed=8)
    spec, tp, r = L.spec, 2, 1
    x = L.exact["x"]
    sh = L.shard(tp, r)
    kv = sh.kv_cache(B, S + steps)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kv)
    pre = O.attn_stage(x[:, :S], L.W, spec, tp, r)
    kc, vc = pre["k"], pre["v"]
    for i in range(steps):
        xi = L.dev["x"][:, S + i].contiguous()
        p = sh.decode(ATTN, xi, kv, out=nan_like((B, 1024)))
        torch.cuda.synchronize()
        ref = O.decode_attn_stage(x[:, S + i], kc, vc, L.W, spec, tp, r)
        assert_close(to_np(p), ref["partial"], f"decode attn partial step {i}", "bf16")
        assert kv.length == S + i + 1
        k, v = kv.read()
        assert_close(to_np(k)[:, :, S + i], ref["k_new"], f"appended k step {i}", "bf16")
        assert_close(to_np(v)[:, :, S + i], ref["v_new"], f"appended v step {i}", "bf16")
        kc = np.concatenate([kc, ref["k_new"][:, :, None]], axis=2)
        vc = np.concatenate([vc, ref["v_new"][:, :, None]], axis=2)
    h = synth.to_storage(synth.draw_normal((B, 1024), 9), "bf16")
    pm = sh.decode(MLP, h.cuda(), out=nan_like((B, 1024)))
    torch.cuda.synchronize()
    ref = O.mlp_stage(h.float().numpy()[:, None], L.W, spec, tp, r)
    assert_close(to_np(pm), ref["partial"][:, 0], "decode mlp partial", "bf16")


@pytest.mark.parametrize("hidden,heads,kv,ffn,tp,B", [
    (768, 6, 6, 6144, 1, 2),      # K = 768 and 6144: 1 and 3 chunks of 2048 per thread
    (512, 4, 2, 11008, 1, 4),     # K = 11008: 6 chunks (8-chunk variant, ragged)
    (256, 2, 2, 20480, 1, 1),     # FFN shard 20480 > 16384: decode falls back to the GEMM path
    (2048, 32, 8, 2816, 2, 7),    # 16 local heads, 4 KV heads (G = 4)
    (1024, 8, 4, 5504, 2, 33),    # two 32-sequence column tiles, ragged; down K = 2752 (43 groups of 64)
    (512, 8, 8, 1536, 1, 64),     # the largest split-K batch
])
def test_decode_gemv_shapes(hidden, heads, kv, ffn, tp, B):
    announce(f"bf16 decode shapes hidden={hidden} heads={heads}/{kv} ffn={ffn} t={tp} B={B}")
    S = 70
    L = Layer(hidden, heads, kv, ffn, batch=B, seq=S + 1, gamma_noise=True, seed=21)
    r = tp - 1
    sh = L.shard(tp, r)
    kvc = sh.kv_cache(B, S + 1)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kvc)
    p = sh.decode(ATTN, L.dev["x"][:, S].contiguous(), kvc, out=nan_like((B, hidden)))
    torch.cuda.synchronize()
    pre = O.attn_stage(L.exact["x"][:, :S], L.W, L.spec, tp, r)
    ref = O.decode_attn_stage(L.exact["x"][:, S], pre["k"], pre["v"], L.W, L.spec, tp, r)
    assert_close(to_np(p), ref["partial"], "decode attn partial", "bf16")
    h = synth.to_storage(synth.draw_normal((B, hidden), 22), "bf16")
    pm = sh.decode(MLP, h.cuda(), out=nan_like((B, hidden)))
    torch.cuda.synchronize()
    refm = O.mlp_stage(h.float().numpy()[:, None], L.W, L.spec, tp, r)
    assert_close(to_np(pm), refm["partial"][:, 0], "decode mlp partial", "bf16")


@pytest.mark.parametrize("ch", [16, 32, 64])
@pytest.mark.parametrize("hidden,heads,kv,B,S", [(2048, 32, 8, 3, 200), (1024, 16, 2, 2, 137)])
def test_decode_chunk_sizes(ch, hidden, heads, kv, B, S):
    """Query-group decode attention with each chunk length forced (head dims
    64 and 128; ragged last chunk), against the oracle."""
    from tensor_transformer_layer_tp_amd import set_decode_chunk
    announce(f"decode chunk {ch}: hidden={hidden} heads={heads}/{kv} B={B} S={S}")
    tp, r = 2, 1
    L = Layer(hidden, heads, kv, 2 * hidden, batch=B, seq=S + 1, gamma_noise=True, seed=31)
    sh = L.shard(tp, r)
    kvc = sh.kv_cache(B, S + 1)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kvc)
    try:
        set_decode_chunk(ch)
        p = sh.decode(ATTN, L.dev["x"][:, S].contiguous(), kvc, out=nan_like((B, hidden)))
        torch.cuda.synchronize()
    finally:
        set_decode_chunk(0)
    pre = O.attn_stage(L.exact["x"][:, :S], L.W, L.spec, tp, r)
    ref = O.decode_attn_stage(L.exact["x"][:, S], pre["k"], pre["v"], L.W, L.spec, tp, r)
    assert_close(to_np(p), ref["partial"], f"decode attn partial (chunk {ch})", "bf16")


@pytest.mark.parametrize("L_len", [1023, 70000])
def test_decode_long_cache(L_len):
    """Decode against a cache written directly (seeded bf16 values), long
    enough that the split-KV merge covers more than 1024 chunks of 64."""
    announce(f"bf16 decode over a written cache of {L_len} positions")
    hidden, heads, kvh, B = 256, 4, 2, 2
    L = Layer(hidden, heads, kvh, 512, batch=B, seq=1, gamma_noise=True, seed=23)
    sh = L.shard(1, 0)
    kvc = sh.kv_cache(B, L_len + 1)
    shape = kvc.shape
    kc = synth.to_storage(synth.draw_normal(shape, 24), "bf16")
    vc = synth.to_storage(synth.draw_normal(shape, 25), "bf16")
    kvc.write(kc.cuda(), vc.cuda())
    kvc.length = L_len
    p = sh.decode(ATTN, L.dev["x"][:, 0].contiguous(), kvc, out=nan_like((B, hidden)))
    torch.cuda.synchronize()
    kn = kc.float().numpy()[:, :, :L_len]
    vn = vc.float().numpy()[:, :, :L_len]
    ref = O.decode_attn_stage(L.exact["x"][:, 0], kn, vn, L.W, L.spec, 1, 0)
    assert_close(to_np(p), ref["partial"], "decode attn partial", "bf16")
    o = to_np(sh.debug_tensor("o", (B, heads * 64)))
    assert_close(o, ref["o"].reshape(B, -1), "decode o", "bf16")


@pytest.mark.parametrize("B", [1, 3, 70])   # GEMV, split-K and GEMM projection paths
def test_decode_graph_replay(B):
    """A decode step (ATTN + MLP stage) captured in a HIP graph and replayed
    with new inputs: every replay must equal the same step made by eager
    calls on a twin shard, and the device-resident cache length must advance
    by one per replay.  Eager work and synchronisations run between replays."""
    announce(f"decode step in a HIP graph, B={B}: eager warm-up + 3 replays against eager twins")
    S, hid = 24, 512
    L = Layer(hid, 4, 2, 1024, batch=B, seq=S + 4, gamma_noise=True, seed=31)
    sh_e, sh_g = L.shard(2, 1), L.shard(2, 1)
    kv_e, kv_g = sh_e.kv_cache(B, S + 8), sh_g.kv_cache(B, S + 8)
    pre = L.dev["x"][:, :S].contiguous()
    sh_e.prefill(ATTN, pre, kv_e)
    sh_g.prefill(ATTN, pre, kv_g)
    hs = [synth.to_storage(synth.draw_normal((B, hid), 40 + i), "bf16").cuda() for i in range(4)]
    xbuf = torch.empty((B, hid), dtype=torch.bfloat16, device="cuda")
    hbuf = torch.empty_like(xbuf)
    pa, pm = nan_like((B, hid)), nan_like((B, hid))

    def step():
        sh_g.decode(ATTN, xbuf, kv_g, out=pa)
        sh_g.decode(MLP, hbuf, out=pm)

    def eager(i):
        pe = sh_e.decode(ATTN, L.dev["x"][:, S + i].contiguous(), kv_e)
        me = sh_e.decode(MLP, hs[i])
        return pe, me

    # step 0 eagerly on both (sizes the workspace before capture)
    xbuf.copy_(L.dev["x"][:, S])
    hbuf.copy_(hs[0])
    step()
    pe, me = eager(0)
    torch.cuda.synchronize()
    assert torch.equal(pa, pe) and torch.equal(pm, me)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    assert kv_g.length == S + 1                      # capture executes nothing
    for i in range(1, 4):
        xbuf.copy_(L.dev["x"][:, S + i])
        hbuf.copy_(hs[i])
        g.replay()
        pe, me = eager(i)
        torch.cuda.synchronize()
        assert torch.equal(pa, pe), f"replay {i}: attention partial differs from the eager call"
        assert torch.equal(pm, me), f"replay {i}: MLP partial differs from the eager call"
        assert kv_g.length == S + 1 + i
    kg, vg = kv_g.read()
    ke, ve = kv_e.read()
    torch.cuda.synchronize()
    assert torch.equal(kg, ke) and torch.equal(vg, ve)
    # the eager twin itself against the oracle at the last step
    x = L.exact["x"]
    ref_pre = O.attn_stage(x[:, :S + 3], L.W, L.spec, 2, 1)
    ref = O.decode_attn_stage(x[:, S + 3], ref_pre["k"], ref_pre["v"], L.W, L.spec, 2, 1)
    assert_close(to_np(pe), ref["partial"], "last replayed step vs oracle", "bf16")
    del g


def packed_qkv_rows(spec, tp, r):
    """Original row index (into the concatenation [W_q; W_k; W_v]) of every
    packed Q/K/V row of rank r: the rank's q heads, then its k heads, then
    its v heads; inside a head, packed row p holds dim 32 g + w (w < 32) or
    d/2 + 32 g + w - 32 (w >= 32), g = p // 64, w = p % 64."""
    hb, kb, _ = O.rank_blocks(spec, tp, r)
    d = spec.head_dim
    dims = [32 * (p // 64) + (p % 64) if p % 64 < 32 else d // 2 + 32 * (p // 64) + (p % 64) - 32
            for p in range(d)]
    rows = []
    for base, block in ((0, hb), (spec.heads * d, kb), (spec.heads * d + spec.kv_heads * d, kb)):
        for hd in block:
            rows += [base + hd * d + dm for dm in dims]
    return np.array(rows)


@pytest.mark.parametrize("hidden,heads,kv,ffn,tp,r", [(1024, 8, 4, 2816, 2, 1), (512, 8, 8, 1536, 1, 0)])
def test_fp8_codes_bit_exact(hidden, heads, kv, ffn, tp, r):
    """The E4M3 codes and row scales the library computes at load time equal
    the oracle's, byte for byte, for all four packed projections."""
    from oracle import fp8
    announce(f"fp8 weight codes, hidden={hidden} heads={heads}/{kv} ffn={ffn} t={tp} r={r}")
    L = Layer(hidden, heads, kv, ffn, seed=51)
    from tensor_transformer_layer_tp_amd import Shard
    sh = Shard(hidden, heads, kv, ffn, tp, r, decode_fp8=True)
    sh.load_weights({k: v for k, v in L.dev.items()})
    spec, W = L.spec, L.exact
    _, _, fb = O.rank_blocks(spec, tp, r)
    hb, _, _ = O.rank_blocks(spec, tp, r)
    d, fl = spec.head_dim, ffn // tp
    qkv_all = np.concatenate([W["wq"], W["wk"], W["wv"]])
    up_rows = []
    for j in range(fl // 32):
        up_rows.append(W["w_gate"][fb.start + 32 * j: fb.start + 32 * j + 32])
        up_rows.append(W["w_up"][fb.start + 32 * j: fb.start + 32 * j + 32])
    expect = {
        "qkv": qkv_all[packed_qkv_rows(spec, tp, r)],
        "o": W["wo"][:, hb.start * d: hb.stop * d],
        "up": np.concatenate(up_rows),
        "down": W["w_down"][:, fb.start: fb.stop],
    }
    for name, w in expect.items():
        codes, scales = sh.fp8_weights(name)
        torch.cuda.synchronize()
        ref_codes, ref_scales = fp8.quantize_rows(w)
        assert np.array_equal(scales.cpu().numpy(), ref_scales), f"{name}: row scales differ"
        got = codes.cpu().numpy()
        bad = np.count_nonzero(got != ref_codes)
        assert bad == 0, f"{name}: {bad} of {got.size} codes differ"


@pytest.mark.parametrize("hidden,heads,kv,ffn,tp,r", [
    (1024, 8, 4, 2816, 2, 1),     # fp8 chunks per row: 64 (hidden), 32 (o), 88 (down)
    (4096, 32, 8, 5632, 4, 3),    # 256 chunks per row; GQA 8 heads on 2 KV heads
    (512, 8, 8, 1536, 1, 0),      # head_dim 64
])
def test_fp8_decode_matches_oracle(hidden, heads, kv, ffn, tp, r):
    """Batch-1 decode on the fp8 shard against the oracle with the rank's
    weights replaced by their E4M3 values; batch 3 on the same shard takes
    the bf16 weights and matches the unquantised oracle."""
    from oracle import fp8
    from tensor_transformer_layer_tp_amd import Shard
    announce(f"fp8 decode hidden={hidden} heads={heads}/{kv} ffn={ffn} t={tp} r={r}")
    S = 40
    L = Layer(hidden, heads, kv, ffn, batch=3, seq=S + 1, gamma_noise=True, seed=52)
    sh = Shard(hidden, heads, kv, ffn, tp, r, decode_fp8=True)
    sh.load_weights({k: v for k, v in L.dev.items() if k != "x"})
    spec, x = L.spec, L.exact["x"]
    Wq = fp8.rank_weights(L.W, spec, tp, r)
    kvc = sh.kv_cache(1, S + 1)
    sh.prefill(ATTN, L.dev["x"][:1, :S].contiguous(), kvc)
    p = sh.decode(ATTN, L.dev["x"][:1, S].contiguous(), kvc, out=nan_like((1, hidden)))
    h = synth.to_storage(synth.draw_normal((1, hidden), 53), "bf16")
    pm = sh.decode(MLP, h.cuda(), out=nan_like((1, hidden)))
    torch.cuda.synchronize()
    pre = O.attn_stage(x[:1, :S], L.W, spec, tp, r)            # the cache came from bf16 prefill
    ref = O.decode_attn_stage(x[:1, S], pre["k"], pre["v"], Wq, spec, tp, r)
    assert_close(to_np(p), ref["partial"], "fp8 decode attn partial", "bf16")
    refm = O.mlp_stage(h.float().numpy()[:, None], Wq, spec, tp, r)
    assert_close(to_np(pm), refm["partial"][:, 0], "fp8 decode mlp partial", "bf16")
    # the quantisation is visible: the unquantised oracle differs by more than rounding
    ref_bf = O.mlp_stage(h.float().numpy()[:, None], L.W, spec, tp, r)
    assert np.abs(ref_bf["partial"][:, 0] - refm["partial"][:, 0]).max() > 1e-3
    # batch 3 on the same shard: bf16 weights
    kv3 = sh.kv_cache(3, S + 1)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kv3)
    p3 = sh.decode(ATTN, L.dev["x"][:, S].contiguous(), kv3, out=nan_like((3, hidden)))
    torch.cuda.synchronize()
    pre3 = O.attn_stage(x[:, :S], L.W, spec, tp, r)
    ref3 = O.decode_attn_stage(x[:, S], pre3["k"], pre3["v"], L.W, spec, tp, r)
    assert_close(to_np(p3), ref3["partial"], "batch-3 decode on the fp8 shard", "bf16")


@pytest.mark.parametrize("hidden,heads,kv,ffn,B,bs", [
    (1024, 8, 4, 2816, 3, 16),    # split-K projections, GQA (G = 2), 16-position blocks
    (1024, 8, 8, 2816, 1, 32),    # GEMV, one query head per KV head
    (512, 8, 4, 1536, 70, 64),    # GEMM projection path, head_dim 64
])
def test_paged_cache_matches_contiguous(hidden, heads, kv, ffn, B, bs):
    """Prefill into a paged cache with a scrambled block table, then decode
    steps: every partial equals the contiguous cache's bit for bit, and the
    pages gathered through the table hold the contiguous cache's rows."""
    announce(f"paged KV cache B={B} block {bs}, heads {heads}/{kv}")
    S, steps, tp, r = 40, 3, 2, 1
    L = Layer(hidden, heads, kv, ffn, batch=B, seq=S + steps, gamma_noise=True, seed=71)
    sh = L.shard(tp, r)
    cap = S + steps + 5
    mb = -(-cap // bs)
    nblocks = B * mb + 7
    perm = np.random.default_rng(72).permutation(nblocks)[:B * mb].reshape(B, mb)
    kvc = sh.kv_cache(B, cap)
    kvp = sh.kv_cache_paged(B, cap, bs, nblocks)
    kvp.set_block_table(perm)
    pre = L.dev["x"][:, :S].contiguous()
    a = sh.prefill(ATTN, pre, kvc).clone()
    b = sh.prefill(ATTN, pre, kvp).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for i in range(steps):
        xi = L.dev["x"][:, S + i].contiguous()
        pc = sh.decode(ATTN, xi, kvc).clone()
        pp = sh.decode(ATTN, xi, kvp).clone()
        torch.cuda.synchronize()
        assert torch.equal(pc, pp), f"decode step {i}: paged partial differs"
    assert kvp.length == S + steps
    kc, vc = kvc.read()
    kp, vp = kvp.read()
    torch.cuda.synchronize()
    n = S + steps
    for bb in range(B):
        for p in sorted({0, min(bs - 1, n - 1), min(bs, n - 1), n - 1}):
            blk, off = perm[bb, p // bs], p % bs
            assert torch.equal(kp[blk, :, off], kc[bb, :, p]) and torch.equal(vp[blk, :, off], vc[bb, :, p])
    # the contiguous twin against the oracle at the last step
    x = L.exact["x"]
    ref_pre = O.attn_stage(x[:, :S + steps - 1], L.W, L.spec, tp, r)
    ref = O.decode_attn_stage(x[:, S + steps - 1], ref_pre["k"], ref_pre["v"], L.W, L.spec, tp, r)
    assert_close(to_np(pp), ref["partial"], "paged decode vs oracle", "bf16")


def test_decode_equals_prefill_row():
    """Same math both ways: decode of token L after a prefill of L tokens
    equals row L of a prefill over L+1 tokens (GPU against GPU, then both
    against the oracle)."""
    announce("bf16 decode vs prefill row consistency")
    L = Layer(512, 4, 2, 1024, batch=2, seq=65, seed=10)
    sh = L.shard(2, 0)
    full = sh.prefill(ATTN, L.dev["x"]).clone()
    kv = sh.kv_cache(2, 80)
    sh.prefill(ATTN, L.dev["x"][:, :64].contiguous(), kv)
    dec = sh.decode(ATTN, L.dev["x"][:, 64].contiguous(), kv)
    torch.cuda.synchronize()
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, 2, 0)
    assert_close(to_np(dec), ref["partial"][:, 64], "decode row", "bf16")
    assert_close(to_np(full[:, 64]), ref["partial"][:, 64], "prefill row", "bf16")
    assert np.abs(to_np(dec) - to_np(full[:, 64])).max() < 0.05


def test_f32_decode():
    announce("fp32 decode B=2 after prefill 20")
    L = Layer(256, 4, 4, 512, dtype="f32", batch=2, seq=21, seed=11, gamma_noise=True)
    sh = L.shard(2, 1)
    kv = sh.kv_cache(2, 32)
    sh.prefill(ATTN, L.dev["x"][:, :20].contiguous(), kv)
    p = sh.decode(ATTN, L.dev["x"][:, 20].contiguous(), kv)
    torch.cuda.synchronize()
    pre = O.attn_stage(L.exact["x"][:, :20], L.W, L.spec, 2, 1)
    ref = O.decode_attn_stage(L.exact["x"][:, 20], pre["k"], pre["v"], L.W, L.spec, 2, 1)
    assert_close(to_np(p), ref["partial"], "f32 decode partial", "f32")


def test_kv_full_and_errors():
    announce("KV-cache capacity errors")
    L = Layer(512, 4, 4, 768, batch=1, seq=6, seed=12)
    sh = L.shard(1, 0)
    kv = sh.kv_cache(1, 4)
    with pytest.raises(TPError) as e:
        sh.prefill(ATTN, L.dev["x"], kv)           # 6 tokens > capacity 4
    assert e.value.status == TP_E_KV_FULL
    sh.prefill(ATTN, L.dev["x"][:, :4].contiguous(), kv)
    with pytest.raises(TPError) as e:
        sh.decode(ATTN, L.dev["x"][:, 4].contiguous(), kv)
    assert e.value.status == TP_E_KV_FULL
    with pytest.raises(TPError):
        sh.decode(ATTN, L.dev["x"][:, 4].expand(2, 512).contiguous(), kv)   # batch mismatch
    torch.cuda.synchronize()


def test_empty_inputs():
    """Zero sequences or zero tokens: the forward calls refuse them before any
    launch (TP_E_ARG; the output buffer and the cache length stay as they
    were), and a reduce over zero elements does nothing, called through the C
    ABI directly with valid buffers."""
    import ctypes as C
    from tensor_transformer_layer_tp_amd import _native as N
    announce("empty inputs")
    L = Layer(512, 4, 4, 768, batch=1, seq=8, seed=15)
    sh = L.shard(2, 0)
    kv = sh.kv_cache(1, 16)
    sh.prefill(ATTN, L.dev["x"], kv)
    torch.cuda.synchronize()
    assert kv.length == 8
    lib = N.lib()
    out = torch.full((1, 8, 512), 7.0, device="cuda")
    xp, op = C.c_void_p(L.dev["x"].data_ptr()), C.c_void_p(out.data_ptr())
    assert lib.tp_shard_forward_prefill(sh._h, ATTN, xp, 1, 0, kv._h, op, None) == N.TP_E_ARG
    assert lib.tp_shard_forward_prefill(sh._h, ATTN, xp, 0, 8, kv._h, op, None) == N.TP_E_ARG
    assert lib.tp_shard_forward_prefill(sh._h, MLP, xp, 1, 0, None, op, None) == N.TP_E_ARG
    assert lib.tp_shard_forward_decode(sh._h, ATTN, xp, 0, kv._h, op, None) == N.TP_E_ARG
    assert lib.tp_shard_forward_decode(sh._h, MLP, xp, 0, None, op, None) == N.TP_E_ARG
    res = torch.full((4,), 3.0, dtype=torch.bfloat16, device="cuda")
    red = torch.full((4,), 5.0, dtype=torch.bfloat16, device="cuda")
    parts = (C.c_void_p * 2)(out.data_ptr(), out.data_ptr())
    assert lib.tp_partial_reduce(parts, 2, C.c_void_p(res.data_ptr()), C.c_void_p(red.data_ptr()), 0,
                                 N.TP_BF16, None) == N.TP_OK
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)) and bool(torch.all(red == 5.0))
    assert kv.length == 8


# ---------------------------------------------------------------- sequence-parallel variant

@pytest.mark.parametrize("tp,B,S", [(2, 2, 64), (4, 1, 96)])
def test_sequence_parallel_chain(tp, B, S):
    """All ranks of the sequence-parallel flow: per-rank norms of token rows,
    all-gather, stages without their norm, reduce-scatter.  Against the
    oracle's sequence-parallel layer, and bit for bit against the plain GPU
    path (the same kernels on the same values)."""
    from oracle import sp
    announce(f"sequence-parallel chain t={tp} B={B} S={S}")
    hid = 1024
    L = Layer(hid, 8, 4, 2816, batch=B, seq=S, gamma_noise=True, seed=61)
    T, n = B * S, B * S // tp
    shards = [L.shard(tp, r) for r in range(tp)]
    xf = L.dev["x"].reshape(T, hid)
    xs = [xf[r * n:(r + 1) * n].contiguous() for r in range(tp)]
    n1 = all_gather([shards[r].norm(1, xs[r]) for r in range(tp)]).reshape(B, S, hid)
    pa = [sh.prefill(ATTN | PRENORM, n1, out=nan_like((B, S, hid))) for sh in shards]
    hs = [partial_reduce_scatter(pa, r, xs[r]) for r in range(tp)]
    n2 = all_gather([shards[r].norm(2, hs[r]) for r in range(tp)]).reshape(B, S, hid)
    pm = [sh.prefill(MLP | PRENORM, n2, out=nan_like((B, S, hid))) for sh in shards]
    ys = [partial_reduce_scatter(pm, r, hs[r]) for r in range(tp)]
    torch.cuda.synchronize()
    ref = sp.layer_sp(L.exact["x"], L.W, L.spec, tp)
    x_rows = [L.exact["x"].reshape(T, hid)[r * n:(r + 1) * n] for r in range(tp)]
    for r in range(tp):
        assert_close(to_np(n1).reshape(T, hid)[r * n:(r + 1) * n], ref["n1"][r], f"n1 rows r{r}", "bf16")
        assert_close(to_np(pa[r]), ref["attn"][r]["partial"], f"attn partial r{r}", "bf16")
        assert_close(to_np(hs[r]), ref["h"][r], f"h rows r{r}", "bf16",
                     sum_magnitude(x_rows[r], [a["partial"].reshape(T, hid)[r * n:(r + 1) * n] for a in ref["attn"]]))
    y = np.concatenate([to_np(v) for v in ys])
    rel = np.linalg.norm(y - np.concatenate(ref["y"])) / np.linalg.norm(np.concatenate(ref["y"]))
    assert rel <= 1e-2, f"sequence-parallel y: relative Frobenius error {rel:.3g}"
    # the plain flow on the GPU gives the same bits
    pa_plain = [sh.prefill(ATTN, L.dev["x"], out=nan_like((B, S, hid))) for sh in shards]
    h_plain = partial_reduce(pa_plain, residual=L.dev["x"])
    pm_plain = [sh.prefill(MLP, h_plain, out=nan_like((B, S, hid))) for sh in shards]
    y_plain = partial_reduce(pm_plain, residual=h_plain)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(hs), h_plain.reshape(T, hid))
    assert torch.equal(torch.cat(ys), y_plain.reshape(T, hid))


# ---------------------------------------------------------------- full-size workloads

def test_7b_t2_prefill_full():
    """hidden 4096, 32 heads x 128, SwiGLU 11008, t=2, B=1, S=2048: both
    ranks and both reduces, every element of every tensor."""
    announce("7B-shaped t=2 prefill B=1 S=2048, both ranks, full compare")
    w = synth.WORKLOADS["7b-t2-prefill"]
    L = Layer(w.hidden, w.heads, w.kv_heads, w.ffn, batch=w.batch, seq=w.seq, seed=0)
    run_chain(L, 2, 1, 2048)


def test_7b_t4_decode_full():
    """rank 0 of t=4, decode B=1 against a 1024-position N(0,1) cache."""
    announce("7B-shaped t=4 decode B=1 L=1024, rank 0")
    w = synth.WORKLOADS["7b-t4-decode"]
    L = Layer(w.hidden, w.heads, w.kv_heads, w.ffn, kv_len=w.kv_len, decode_batch=1, seed=0)
    sh = L.shard(4, 0)
    kv = sh.kv_cache(1, w.kv_len + 8)
    kc = rank_cache(L.exact["k_cache"], L.spec, 4, 0)
    vc = rank_cache(L.exact["v_cache"], L.spec, 4, 0)
    kfull = torch.zeros(kv.shape, dtype=torch.bfloat16)
    vfull = torch.zeros(kv.shape, dtype=torch.bfloat16)
    kfull[:, :, :w.kv_len] = torch.from_numpy(kc).to(torch.bfloat16)
    vfull[:, :, :w.kv_len] = torch.from_numpy(vc).to(torch.bfloat16)
    kv.write(kfull.cuda(), vfull.cuda())
    kv.length = w.kv_len
    p = sh.decode(ATTN, L.dev["x_dec"], kv, out=nan_like((1, w.hidden)))
    torch.cuda.synchronize()
    ref = O.decode_attn_stage(L.exact["x_dec"], kc, vc, L.W, L.spec, 4, 0)
    assert_close(to_np(p), ref["partial"], "7B decode attn partial", "bf16")
    h = synth.to_storage(synth.draw_normal((1, w.hidden), 21), "bf16")
    pm = sh.decode(MLP, h.cuda(), out=nan_like((1, w.hidden)))
    torch.cuda.synchronize()
    refm = O.mlp_stage(h.float().numpy()[:, None], L.W, L.spec, 4, 0)
    assert_close(to_np(pm), refm["partial"][:, 0], "7B decode mlp partial", "bf16")


@pytest.fixture(scope="module")
def layer70b():
    w = synth.WORKLOADS["70b-t8-prefill"]
    return Layer(w.hidden, w.heads, w.kv_heads, w.ffn, batch=w.batch, seq=w.seq,
                 kv_len=4096, decode_batch=1, seed=0)


def test_70b_t8_prefill_sampled(layer70b):
    """rank 0 of t=8 (8 query heads, 1 KV head), B=4, S=4096: the full GPU
    output, checked on sampled rows of every batch element (the oracle
    computes the keys and values of the whole prefix) and on the whole KV
    cache."""
    announce("70B-shaped t=8 prefill B=4 S=4096 rank 0, sampled rows")
    L = layer70b
    B, S = 4, 4096
    sh = L.shard(8, 0)
    kv = sh.kv_cache(B, S)
    p = sh.prefill(ATTN, L.dev["x"], kv, out=nan_like((B, S, 8192)))
    torch.cuda.synchronize()
    pg = to_np(p)
    assert np.isfinite(pg).all()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 2047, 2048, 4094, 4095],
                                     rng.integers(0, S, 22)]))
    ref = O.attn_stage_rows(L.exact["x"], L.W, L.spec, 8, 0, rows)
    assert_close(pg[:, rows], ref["partial"], "70B attn partial (sampled rows)", "bf16")
    k, v = kv.read()
    assert_close(to_np(k), ref["k"], "70B K cache", "bf16")
    assert_close(to_np(v), ref["v"], "70B V cache", "bf16")
    h = synth.to_storage(synth.draw_normal((B, S, 8192), 31), "bf16")
    pm = sh.prefill(MLP, h.cuda(), out=nan_like((B, S, 8192)))
    torch.cuda.synchronize()
    pmg = to_np(pm)
    assert np.isfinite(pmg).all()
    refm = O.mlp_stage_rows(h.float().numpy(), L.W, L.spec, 8, 0, rows)
    assert_close(pmg[:, rows], refm["partial"], "70B mlp partial (sampled rows)", "bf16")


def test_70b_t8_decode_full(layer70b):
    announce("70B-shaped t=8 decode B=1 L=4096 rank 0")
    L = layer70b
    sh = L.shard(8, 0)
    kv = sh.kv_cache(1, 4096 + 16)
    kc = rank_cache(L.exact["k_cache"], L.spec, 8, 0)
    vc = rank_cache(L.exact["v_cache"], L.spec, 8, 0)
    kfull = torch.zeros(kv.shape, dtype=torch.bfloat16)
    vfull = torch.zeros(kv.shape, dtype=torch.bfloat16)
    kfull[:, :, :4096] = torch.from_numpy(kc).to(torch.bfloat16)
    vfull[:, :, :4096] = torch.from_numpy(vc).to(torch.bfloat16)
    kv.write(kfull.cuda(), vfull.cuda())
    kv.length = 4096
    p = sh.decode(ATTN, L.dev["x_dec"], kv, out=nan_like((1, 8192)))
    torch.cuda.synchronize()
    ref = O.decode_attn_stage(L.exact["x_dec"], kc, vc, L.W, L.spec, 8, 0)
    assert_close(to_np(p), ref["partial"], "70B decode attn partial", "bf16")
    h = synth.to_storage(synth.draw_normal((1, 8192), 41), "bf16")
    pm = sh.decode(MLP, h.cuda(), out=nan_like((1, 8192)))
    torch.cuda.synchronize()
    refm = O.mlp_stage(h.float().numpy()[:, None], L.W, L.spec, 8, 0)
    assert_close(to_np(pm), refm["partial"][:, 0], "70B decode mlp partial", "bf16")


# ---------------------------------------------------------------- every GEMM tile configuration

@pytest.mark.parametrize("ffn", [2816, 2688])   # FFN shard 1408 (22 K-steps of 64) and 1344 (21: odd)
def test_every_gemm_config(ffn):
    """Each projection tile configuration (register-staged and DMA-ring
    variants), forced in turn, on a ragged token count, against the oracle."""
    from tensor_transformer_layer_tp_amd import set_gemm_config
    from tensor_transformer_layer_tp_amd import _native as N
    announce(f"every GEMM configuration, ffn={ffn}")
    L = Layer(1024, 8, 4, ffn, batch=1, seq=300, gamma_noise=True, seed=13)
    h = synth.to_storage(synth.draw_normal((1, 300, 1024), 14), "bf16")
    ref_a = O.attn_stage(L.exact["x"], L.W, L.spec, 2, 1)
    ref_m = O.mlp_stage(h.float().numpy(), L.W, L.spec, 2, 1)
    sh = L.shard(2, 1)
    n_cfg = 17
    assert N.lib().tp_tune_set_gemm_config(n_cfg) == N.TP_E_ARG   # the table has exactly n_cfg entries
    try:
        for cfg in range(n_cfg):
            set_gemm_config(cfg)
            pa = sh.prefill(ATTN, L.dev["x"], out=nan_like((1, 300, 1024)))
            pm = sh.prefill(MLP, h.cuda(), out=nan_like((1, 300, 1024)))
            torch.cuda.synchronize()
            assert_close(to_np(pa), ref_a["partial"], f"cfg {cfg} attn partial", "bf16")
            assert_close(to_np(pm), ref_m["partial"], f"cfg {cfg} mlp partial", "bf16")
    finally:
        set_gemm_config(-1)
