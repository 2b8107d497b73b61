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

from helpers import Layer, assert_bf16_close, assert_close, rank_cache, report, to_np

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


def nan_like(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def run_chain(layer: Layer, tp: int, B: int, S: int, check_kv=True):
    """All tp ranks of a prefill: ATTN stages, reduce, MLP stages, reduce,
    chained on the GPU exactly as a caller runs them (the MLP stages take
    the GPU's own h).

    Every GPU tensor is compared element by element with the oracle applied
    to the same inputs: the ATTN partials and the K/V cache on x; h with the
    oracle's reduce of the GPU's own partials (fp32 values, exact) and with
    the oracle's chain; the MLP partials with the oracle's MLP stage on the
    GPU's h (bf16 values, exactly representable); y with the oracle's reduce
    of those oracle partials plus the GPU's h, and with the oracle's reduce
    of the GPU's own MLP partials.  The whole GPU chain against the whole
    oracle chain is compared element by element for fp32 and reported as a
    diagnostic for bf16 (its norm-relative error is bounded)."""
    dt = layer.dtype
    spec = layer.spec
    x_dev = layer.dev["x"]
    hid = spec.hidden
    ref = O.layer(layer.exact["x"], layer.W, spec, t=tp)
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
    h_np = to_np(h)
    assert_close(h_np, O.reduce([to_np(p) for p in pa], layer.exact["x"], spec), "h (reduce of the GPU partials)", dt)
    assert_close(h_np, ref["h"], "h", dt)
    # the MLP stages on the GPU's own h
    pm = [sh.prefill(MLP, h, out=nan_like((B, S, hid))) for sh in shards]
    y = partial_reduce(pm, residual=h)
    torch.cuda.synchronize()
    ref_m = [O.mlp_stage(h_np, layer.W, spec, tp, r) for r in range(tp)]
    for r in range(tp):
        assert_close(to_np(pm[r]), ref_m[r]["partial"], f"mlp partial r{r} (on the GPU's h)", dt)
    y_np = to_np(y)
    assert_close(y_np, O.reduce([m["partial"] for m in ref_m], h_np, spec), "y (chained)", dt)
    assert_close(y_np, O.reduce([to_np(p) for p in pm], h_np, spec), "y (reduce of the GPU partials)", dt)
    # end to end against the oracle's own chain
    if dt == "f32":
        assert_close(y_np, ref["y"], "y (oracle chain)", dt)
    else:
        rel, _ = report(y_np, ref["y"], f"y end to end vs the oracle chain, t={tp} B={B} S={S}")
        assert rel <= 1e-2, f"y end to end: norm-relative error {rel:.3g}"
    return shards, kvs


def sampled_chain(W_dev, W_np, spec, tp, x_dev, x_np, rows, check_kv=True, gemm_plans=None):
    """A full-size prefill chain (every rank, both reduces) run in full on
    the GPU and checked on sampled token rows of the selected sequences.

    x_np maps a sequence index b to its exact input [S, hidden]; the oracle
    computes the keys and values of the whole prefix of those sequences and
    the stage outputs at ``rows``.  Every check uses the same inputs on both
    sides, as in run_chain: the reduce on the GPU's partial rows, the MLP
    stages on the GPU's h rows."""
    from tensor_transformer_layer_tp_amd import Shard
    B, S, hid = (int(v) for v in x_dev.shape)
    bsel = sorted(x_np)
    xs = np.stack([x_np[b] for b in bsel])               # [len(bsel), S, hid]
    shards = []
    for r in range(tp):
        sh = Shard(spec.hidden, spec.heads, spec.kv_heads, spec.ffn, tp, r)
        sh.load_weights(W_dev)
        shards.append(sh)
    kvs = [sh.kv_cache(B, S) for sh in shards] if check_kv else [None] * tp
    pa = [sh.prefill(ATTN, x_dev, kv, out=nan_like((B, S, hid))) for sh, kv in zip(shards, kvs)]
    h = partial_reduce(pa, residual=x_dev)
    torch.cuda.synchronize()
    pa_rows = [to_np(p[bsel][:, rows]) for p in pa]
    h_rows = to_np(h[bsel][:, rows])
    for p in pa:
        assert bool(torch.isfinite(p).all()), "attention partial: non-finite values (unwritten)"
    del pa
    refa = [O.attn_stage_rows(xs, W_np, spec, tp, r, rows) for r in range(tp)]
    for r in range(tp):
        assert_bf16_close(pa_rows[r], refa[r]["partial"], f"attn partial r{r} (sampled rows)")
        if check_kv:
            k, v = kvs[r].read()
            torch.cuda.synchronize()
            assert_bf16_close(to_np(k[bsel]), refa[r]["k"], f"K cache r{r} (selected sequences)")
            assert_bf16_close(to_np(v[bsel]), refa[r]["v"], f"V cache r{r} (selected sequences)")
            del k, v
            assert kvs[r].length == S
            kvs[r].close()
    x_rows = xs[:, rows]
    assert_bf16_close(h_rows, O.reduce(pa_rows, x_rows, spec), "h rows (reduce of the GPU partials)")
    assert_bf16_close(h_rows, O.reduce([a["partial"] for a in refa], x_rows, spec), "h rows")
    pm = [sh.prefill(MLP, h, out=nan_like((B, S, hid))) for sh in shards]
    y = partial_reduce(pm, residual=h)
    torch.cuda.synchronize()
    pm_rows = [to_np(p[bsel][:, rows]) for p in pm]
    y_rows = to_np(y[bsel][:, rows])
    for p in pm:
        assert bool(torch.isfinite(p).all()), "MLP partial: non-finite values (unwritten)"
    del pm, h, y
    refm = [O.mlp_stage(h_rows, W_np, spec, tp, r) for r in range(tp)]
    for r in range(tp):
        assert_bf16_close(pm_rows[r], refm[r]["partial"], f"mlp partial r{r} (sampled rows, on the GPU's h)")
    assert_bf16_close(y_rows, O.reduce([m["partial"] for m in refm], h_rows, spec), "y rows (chained)")
    assert_bf16_close(y_rows, O.reduce(pm_rows, h_rows, spec), "y rows (reduce of the GPU partials)")
    for sh in shards:
        sh.close()


def sample_rows(S, seed, n=62):
    """First, last and n random token rows (sorted, distinct)."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, n)]))


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
    assert_close(to_np(out), want, "reduce", dtype)
    out2 = partial_reduce(parts, residual=None, dtype=dtype)
    want2 = O.reduce([p.astype(np.float32) for p in parts64], np.zeros(n), spec)
    assert_close(to_np(out2), want2, "reduce no residual", dtype)


@pytest.mark.parametrize("hidden,heads,kv,t,rows,dtype", [
    (512, 4, 4, 2, 300, "bf16"),      # two 8-value chunks per thread (the norm's MAXC 2), ragged rows
    (1536, 12, 3, 3, 77, "bf16"),     # a run-time rank count (the generic summation loop)
    (4096, 32, 32, 1, 5, "bf16"),     # one rank: the reduce is a cast plus the residual
    (8192, 64, 8, 8, 257, "bf16"),    # the 70B width, eight ranks (MAXC 4)
    (9216, 72, 8, 2, 33, "bf16"),     # wider than the fused kernel: reduce, then norm
    (512, 4, 4, 2, 40, "f32"),        # the fp32 path: reduce, then norm
])
def test_reduce_norm(hidden, heads, kv, t, rows, dtype):
    """tp_shard_reduce_norm (the reduce with the next stage's RMSNorm) bit for
    bit against tp_partial_reduce followed by tp_shard_norm, and against the
    oracle: the reduce of the same partials, then the norm of the stored
    result, with both gains."""
    announce(f"reduce + RMSNorm hidden={hidden} t={t} rows={rows} {dtype}")
    L = Layer(hidden, heads, kv, 512 * t, dtype=dtype, seq=0, gamma_noise=True, seed=41)
    sh = L.shard(t, 0)
    parts64 = [synth.draw_normal((rows, hidden), 42 + r, 3.0) for r in range(t)]
    parts = [torch.from_numpy(p).cuda() for p in parts64]
    res = synth.to_storage(synth.draw_normal((rows, hidden), 50), dtype)
    for which, norm_ref in ((1, O.norm1), (2, O.norm2)):
        out, nout = sh.reduce_norm(which, parts, residual=res.cuda())
        h = partial_reduce(parts, residual=res.cuda())
        n = sh.norm(which, h)
        torch.cuda.synchronize()
        assert torch.equal(out, h), "fused reduce differs from tp_partial_reduce"
        assert torch.equal(nout, n), "fused norm differs from tp_shard_norm"
        h_np = to_np(out)
        assert_close(h_np, O.reduce([p.astype(np.float64) for p in parts64], res.float().numpy(), L.spec),
                     f"reduce (which={which})", dtype)
        assert_close(to_np(nout), norm_ref(h_np, L.W, L.spec), f"norm of the reduce (which={which})", dtype)
    # no residual
    out, nout = sh.reduce_norm(2, parts)
    torch.cuda.synchronize()
    assert_close(to_np(out), O.reduce([p.astype(np.float64) for p in parts64], np.zeros((rows, hidden)), L.spec),
                 "reduce without a residual", dtype)


def test_fused_norm_chain_equals_plain_chain():
    """A layer chained through the fused reduce-norms (norm of x once, then
    ATTN|PRENORM, reduce+norm2, MLP|PRENORM, reduce+norm1 of y) gives the
    plain chain's partials, h and y bit for bit, and the norm of y that the
    next layer's ATTN stage would compute."""
    announce("layer through the fused reduce-norms vs the plain chain, t=2")
    B, S, hid = 2, 96, 1024
    L = Layer(hid, 8, 4, 2816, batch=B, seq=S, gamma_noise=True, seed=43)
    shards = [L.shard(2, r) for r in range(2)]
    x = L.dev["x"]
    pa = [sh.prefill(ATTN, x) for sh in shards]
    h = partial_reduce(pa, residual=x)
    pm = [sh.prefill(MLP, h) for sh in shards]
    y = partial_reduce(pm, residual=h)
    n1 = shards[0].norm(1, x)
    pa_f = [sh.prefill(ATTN | PRENORM, n1) for sh in shards]
    h_f, n2_f = shards[0].reduce_norm(2, pa_f, residual=x)
    pm_f = [sh.prefill(MLP | PRENORM, n2_f) for sh in shards]
    y_f, n1_next = shards[0].reduce_norm(1, pm_f, residual=h_f)
    n1_y = shards[0].norm(1, y)
    torch.cuda.synchronize()
    for a, b in zip(pa + pm, pa_f + pm_f):
        assert torch.equal(a, b)
    assert torch.equal(h, h_f) and torch.equal(y, y_f) and torch.equal(n1_y, n1_next)


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


@pytest.mark.parametrize("kern", [1, 2])
@pytest.mark.parametrize("kg", [1, 2])
@pytest.mark.parametrize("hidden,heads,kv,S", [(1024, 8, 4, 300), (512, 8, 2, 130), (1024, 8, 2, 1000),
                                               (512, 4, 4, 64), (1024, 8, 8, 1)])
def test_attention_key_groups(kern, kg, hidden, heads, kv, S):
    """Prefill attention with one group of waves over every key block and
    with two groups over alternate key blocks whose softmax states merge,
    forced in turn, each on the one-stage kernel (1) and on the pipelined
    kernel (2): head dims 128 and 64, GQA and MHA, ragged S, one key block, a
    single token, against the oracle's attention output."""
    from tensor_transformer_layer_tp_amd import set_attn_groups, set_attn_kernel
    announce(f"attention kernel {kern} key groups kg={kg} hidden={hidden} heads={heads}/{kv} S={S}")
    t, r, B = 2, 1, 2
    L = Layer(hidden, heads, kv, 2 * hidden, batch=B, seq=S, gamma_noise=True, seed=21)
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, t, r)
    sh = L.shard(t, r)
    hl, d = heads // t, hidden // heads
    try:
        set_attn_groups(kg)
        set_attn_kernel(kern)
        sh.prefill(ATTN, L.dev["x"])
        o = sh.debug_tensor("o", (B * S, hl * d))
        torch.cuda.synchronize()
    finally:
        set_attn_groups(0)
        set_attn_kernel(0)
    assert_close(to_np(o), ref["o"].transpose(0, 2, 1, 3).reshape(B * S, hl * d),
                 f"attention o kernel {kern} kg={kg}", "bf16")


@pytest.mark.parametrize("S", [65, 128, 129, 192, 257])
@pytest.mark.parametrize("hidden,heads,kv", [(1024, 8, 8), (1024, 8, 2), (1024, 16, 2), (512, 8, 4)])
def test_attention_block_counts(hidden, heads, kv, S):
    """The default prefill attention over sequence lengths that give each
    query block one, two, three or more key blocks per key group (odd and
    even trip counts of the two-blocks-per-trip loop, ragged last blocks),
    head dims 128 and 64, MHA and GQA up to four query heads per KV head,
    against the oracle's attention output."""
    announce(f"attention block counts hidden={hidden} heads={heads}/{kv} S={S}")
    t, r, B = 2, 0, 2
    L = Layer(hidden, heads, kv, 2 * hidden, batch=B, seq=S, gamma_noise=True, seed=31)
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, t, r)
    sh = L.shard(t, r)
    hl, d = heads // t, hidden // heads
    sh.prefill(ATTN, L.dev["x"])
    o = sh.debug_tensor("o", (B * S, hl * d))
    torch.cuda.synchronize()
    assert_close(to_np(o), ref["o"].transpose(0, 2, 1, 3).reshape(B * S, hl * d), "attention o", "bf16")


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


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("ch", [16, 32, 64])
@pytest.mark.parametrize("hidden,heads,kv,B,S", [(2048, 32, 8, 3, 200), (1024, 16, 2, 2, 137), (1024, 8, 8, 2, 150)])
def test_decode_chunk_sizes(mode, ch, hidden, heads, kv, B, S):
    """Decode attention with each chunk length forced (head dims 64 and 128;
    query groups of 4 and 8 and one query head per KV head; ragged last
    chunk), with each attention form: one query head per chunk work-group
    and a merge launch (mode 0, the default), the KV-head chunk kernels and a
    merge launch (mode 1), the merge in the same launch (mode 2); against
    the oracle: the attention output o and the partial."""
    from tensor_transformer_layer_tp_amd import set_decode_attn, set_decode_chunk
    announce(f"decode attention mode {mode} chunk {ch}: hidden={hidden} heads={heads}/{kv} B={B} S={S}")
    tp, r = 2, 1
    L = Layer(hidden, heads, kv, 2 * hidden, batch=B, seq=S + 1, gamma_noise=True, seed=31)
    sh = L.shard(tp, r)
    kvc = sh.kv_cache(B, S + 1)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kvc)
    try:
        set_decode_chunk(ch)
        set_decode_attn(mode)
        p = sh.decode(ATTN, L.dev["x"][:, S].contiguous(), kvc, out=nan_like((B, hidden)))
        o = sh.debug_tensor("o", (B, heads // tp * (hidden // heads)))
        torch.cuda.synchronize()
    finally:
        set_decode_chunk(0)
        set_decode_attn(0)
    pre = O.attn_stage(L.exact["x"][:, :S], L.W, L.spec, tp, r)
    ref = O.decode_attn_stage(L.exact["x"][:, S], pre["k"], pre["v"], L.W, L.spec, tp, r)
    assert_close(to_np(o), ref["o"].reshape(B, -1), f"decode o (mode {mode}, chunk {ch})", "bf16")
    assert_close(to_np(p), ref["partial"], f"decode attn partial (mode {mode}, chunk {ch})", "bf16")


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("L_len", [1023, 70000])
def test_decode_long_cache(L_len, mode):
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
    from tensor_transformer_layer_tp_amd import set_decode_attn
    try:
        set_decode_attn(mode)   # 70000 positions: automatic = merge launch; forced: the in-launch merge
        p = sh.decode(ATTN, L.dev["x"][:, 0].contiguous(), kvc, out=nan_like((B, hidden)))
        torch.cuda.synchronize()
    finally:
        set_decode_attn(0)
    kn = kc.float().numpy()[:, :, :L_len]
    vn = vc.float().numpy()[:, :, :L_len]
    ref = O.decode_attn_stage(L.exact["x"][:, 0], kn, vn, L.W, L.spec, 1, 0)
    assert_close(to_np(p), ref["partial"], "decode attn partial", "bf16")
    o = to_np(sh.debug_tensor("o", (B, heads * 64)))
    assert_close(o, ref["o"].reshape(B, -1), "decode o", "bf16")


def _fused_pair(L, tp, r, fp8):
    """Two identical shards (the E4M3 variant with fp8)."""
    def make():
        if not fp8:
            return L.shard(tp, r)
        s = L.spec
        sh = Shard(s.hidden, s.heads, s.kv_heads, s.ffn, tp, r, decode_fp8=True)
        sh.load_weights({k: v for k, v in L.dev.items() if k not in ("x", "k_cache", "v_cache", "x_dec")})
        return sh
    return make(), make()


@pytest.mark.parametrize("dtype,B,tp,r,fp8,res", [
    ("bf16", 1, 2, 1, False, True),    # GEMV epilogue
    ("bf16", 1, 8, 0, False, True),    # eight ranks, own slot first
    ("bf16", 1, 8, 7, True, True),     # E4M3 GEMV, own slot last
    ("bf16", 3, 4, 2, False, False),   # split-K epilogue, no residual
    ("bf16", 70, 2, 0, False, True),   # GEMM path: workspace partial, then the reduce
    ("f32", 2, 2, 1, False, True),     # fp32 shard: workspace partial, then the reduce
])
def test_decode_reduce_equals_two_calls(dtype, B, tp, r, fp8, res):
    """tp_shard_forward_decode_reduce against tp_shard_forward_decode followed
    by tp_partial_reduce with the same other-rank partials: h and y bit for
    bit and the caches bit for bit, for both stages; h also against the
    oracle's reduce of the oracle's decode partial and the same other-rank
    partials."""
    announce(f"decode with the reduce folded in: {dtype} B={B} t={tp} rank {r} fp8={fp8} residual={res}")
    hid, S = 1024, 48
    L = Layer(hid, 16, 8, 4096, dtype=dtype, batch=B, seq=S + 1, gamma_noise=True, seed=51)
    sh_a, sh_b = _fused_pair(L, tp, r, fp8)
    kv_a, kv_b = sh_a.kv_cache(B, S + 4), sh_b.kv_cache(B, S + 4)
    pre = L.dev["x"][:, :S].contiguous()
    sh_a.prefill(ATTN, pre, kv_a)
    sh_b.prefill(ATTN, pre, kv_b)
    x = L.dev["x"][:, S].contiguous()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    oth_a = [torch.randn((B, hid), generator=g, device="cuda") for _ in range(tp)]
    oth_m = [torch.randn((B, hid), generator=g, device="cuda") for _ in range(tp)]
    resid = (lambda t: t) if res else (lambda t: None)
    pa = sh_a.decode(ATTN, x, kv_a)
    h_ref = partial_reduce([pa if j == r else oth_a[j] for j in range(tp)], residual=resid(x), dtype=dtype)
    pm = sh_a.decode(MLP, h_ref)
    y_ref = partial_reduce([pm if j == r else oth_m[j] for j in range(tp)], residual=resid(h_ref), dtype=dtype)
    h = sh_b.decode_reduce(ATTN, x, [None if j == r else oth_a[j] for j in range(tp)], residual=resid(x), kv=kv_b)
    y = sh_b.decode_reduce(MLP, h, [None if j == r else oth_m[j] for j in range(tp)], residual=resid(h))
    torch.cuda.synchronize()
    assert torch.equal(h, h_ref), "h differs from decode + partial_reduce"
    assert torch.equal(y, y_ref), "y differs from decode + partial_reduce"
    ka, va = kv_a.read()
    kb, vb = kv_b.read()
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert kv_b.length == S + 1
    if not fp8:
        pre_o = O.attn_stage(L.exact["x"][:, :S], L.W, L.spec, tp, r)
        ref = O.decode_attn_stage(L.exact["x"][:, S], pre_o["k"], pre_o["v"], L.W, L.spec, tp, r)
        parts = [ref["partial"] if j == r else to_np(oth_a[j]) for j in range(tp)]
        resid_np = L.exact["x"][:, S] if res else np.zeros((B, hid))
        assert_close(to_np(h), O.reduce(parts, resid_np, L.spec), "fused h vs the oracle's reduce", dtype)


@pytest.mark.parametrize("B", [1, 3])
def test_decode_reduce_graph_replay(B):
    """A decode step made of the two fused calls, captured in a HIP graph and
    replayed with new inputs, against eager twins (bit for bit)."""
    announce(f"fused decode step in a HIP graph, B={B}: 3 replays against eager twins")
    S, hid, tp, r = 24, 512, 2, 1
    L = Layer(hid, 4, 2, 1024, batch=B, seq=S + 4, gamma_noise=True, seed=61)
    sh_e, sh_g = L.shard(tp, r), L.shard(tp, r)
    kv_e, kv_g = sh_e.kv_cache(B, S + 8), sh_g.kv_cache(B, S + 8)
    pre = L.dev["x"][:, :S].contiguous()
    sh_e.prefill(ATTN, pre, kv_e)
    sh_g.prefill(ATTN, pre, kv_g)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    oth = [[torch.randn((B, hid), generator=g, device="cuda") for _ in range(tp)] for _ in range(2)]
    xbuf = torch.empty((B, hid), dtype=torch.bfloat16, device="cuda")
    hbuf, ybuf = torch.empty_like(xbuf), torch.empty_like(xbuf)

    def step():
        sh_g.decode_reduce(ATTN, xbuf, oth[0], residual=xbuf, kv=kv_g, out=hbuf)
        sh_g.decode_reduce(MLP, hbuf, oth[1], residual=hbuf, out=ybuf)

    def eager(i):
        h = sh_e.decode_reduce(ATTN, L.dev["x"][:, S + i].contiguous(), oth[0],
                               residual=L.dev["x"][:, S + i].contiguous(), kv=kv_e)
        return h, sh_e.decode_reduce(MLP, h, oth[1], residual=h)

    xbuf.copy_(L.dev["x"][:, S])
    step()
    he, ye = eager(0)
    torch.cuda.synchronize()
    assert torch.equal(hbuf, he) and torch.equal(ybuf, ye)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(1, 4):
        xbuf.copy_(L.dev["x"][:, S + i])
        graph.replay()
        he, ye = eager(i)
        torch.cuda.synchronize()
        assert torch.equal(hbuf, he), f"replay {i}: h differs from the eager call"
        assert torch.equal(ybuf, ye), f"replay {i}: y differs from the eager call"
        assert kv_g.length == S + 1 + i
    del graph


@pytest.mark.parametrize("dtype,tp,r,res,cfg", [
    ("bf16", 2, 1, True, None),        # the planner's tiles (staged epilogue), own slot last
    ("bf16", 8, 0, True, None),        # eight ranks, own slot first
    ("bf16", 4, 2, False, None),       # no residual
    ("bf16", 2, 0, True, 1),           # register-staged 128x128 tile: the per-element epilogue
    ("bf16", 2, 1, True, 14),          # producer/consumer 256x256 (the twelve-wave sum epilogue)
    ("bf16", 8, 3, True, 14),          # ... with eight ranks, own slot in the middle
    ("bf16", 2, 1, True, 15),          # producer/consumer 256x192, eight MFMA waves
    ("bf16", 2, 1, True, 17),          # producer/consumer 256x192, four MFMA waves
    ("bf16", 2, 1, True, 18),          # producer/consumer 256x128, four MFMA waves
    ("bf16", 2, 1, True, "split"),     # two launches over column ranges (the second at column 640)
    ("f32", 2, 1, True, None),         # fp32 shard: workspace partial, then the reduce
])
def test_prefill_reduce_equals_two_calls(dtype, tp, r, res, cfg):
    """tp_shard_forward_prefill_reduce against tp_shard_forward_prefill
    followed by tp_partial_reduce with the same other-rank partials: h and y
    bit for bit and the caches bit for bit, for both stages and on a ragged
    token count; h also against the oracle's reduce of the oracle's partial
    and the same other-rank partials."""
    from tensor_transformer_layer_tp_amd import set_gemm_config, set_gemm_split
    announce(f"prefill with the reduce folded in: {dtype} t={tp} rank {r} residual={res} tiles={cfg}")
    hid, B, S = 1024, 2, 150
    L = Layer(hid, 16, 8, 4096, dtype=dtype, batch=B, seq=S, gamma_noise=True, seed=61)
    sh_a, sh_b = L.shard(tp, r), L.shard(tp, r)
    kv_a, kv_b = sh_a.kv_cache(B, S), sh_b.kv_cache(B, S)
    x = L.dev["x"]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    oth_a = [torch.randn((B, S, hid), generator=g, device="cuda") for _ in range(tp)]
    oth_m = [torch.randn((B, S, hid), generator=g, device="cuda") for _ in range(tp)]
    resid = (lambda t: t) if res else (lambda t: None)
    try:
        if cfg == "split":
            set_gemm_split(14, 16, 640)
        elif cfg is not None:
            set_gemm_config(cfg)
        pa = sh_a.prefill(ATTN, x, kv_a)
        h_ref = partial_reduce([pa if j == r else oth_a[j] for j in range(tp)], residual=resid(x), dtype=dtype)
        pm = sh_a.prefill(MLP, h_ref)
        y_ref = partial_reduce([pm if j == r else oth_m[j] for j in range(tp)], residual=resid(h_ref), dtype=dtype)
        h = sh_b.prefill_reduce(ATTN, x, [None if j == r else oth_a[j] for j in range(tp)], residual=resid(x),
                                kv=kv_b)
        y = sh_b.prefill_reduce(MLP, h, [None if j == r else oth_m[j] for j in range(tp)], residual=resid(h))
        torch.cuda.synchronize()
    finally:
        set_gemm_config(-1)
        set_gemm_split(0, 0, 0)
    assert torch.equal(h, h_ref), "h differs from prefill + partial_reduce"
    assert torch.equal(y, y_ref), "y differs from prefill + partial_reduce"
    ka, va = kv_a.read()
    kb, vb = kv_b.read()
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert kv_b.length == S
    ref = O.attn_stage(L.exact["x"], L.W, L.spec, tp, r)
    parts = [ref["partial"] if j == r else to_np(oth_a[j]) for j in range(tp)]
    resid_np = L.exact["x"] if res else np.zeros((B, S, hid))
    assert_close(to_np(h), O.reduce(parts, resid_np, L.spec), "fused h vs the oracle's reduce", dtype)
    refm = O.mlp_stage(to_np(h), L.W, L.spec, tp, r)
    parts = [refm["partial"] if j == r else to_np(oth_m[j]) for j in range(tp)]
    resid_np = to_np(h) if res else np.zeros((B, S, hid))
    assert_close(to_np(y), O.reduce(parts, resid_np, L.spec), "fused y vs the oracle's reduce", dtype)


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


def test_cache_length_in_stream_order():
    """tp_kv_set_len_async / tp_kv_get_len_stream on a side stream: the length
    set in the stream's order is the one a decode call queued after it on that
    stream appends at, the overflow flag is cleared with it, and the decode
    matches the same step after the synchronous tp_kv_set_len bit for bit."""
    announce("cache length set and read in stream order")
    L = Layer(512, 8, 4, 1024, batch=2, seq=40, gamma_noise=True, seed=71)
    sh_a, sh_b = L.shard(2, 1), L.shard(2, 1)
    kv_a, kv_b = sh_a.kv_cache(2, 48), sh_b.kv_cache(2, 48)
    pre = L.dev["x"][:, :33].contiguous()
    sh_a.prefill(ATTN, pre, kv_a)
    sh_b.prefill(ATTN, pre, kv_b)
    x = L.dev["x"][:, 33].contiguous()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    kv_a.length = 30                       # drop the last three positions
    pa = sh_a.decode(ATTN, x, kv_a)
    with torch.cuda.stream(s):
        kv_b.set_length_async(30, stream=s)
        pb = sh_b.decode(ATTN, x, kv_b, stream=s)
        n = kv_b.length_on(s)
    torch.cuda.synchronize()
    assert n == 31
    assert torch.equal(pa, pb)
    ka, va = kv_a.read()
    kb, vb = kv_b.read()
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert kv_a.length == 31


def test_graph_replay_past_capacity_reports_overflow():
    """A captured decode call replayed once more than the cache holds
    appends nothing and raises the cache's overflow flag: the length query
    reports TP_E_KV_FULL, an eager call on the full cache is refused up
    front, and setting the length clears the flag."""
    announce("decode replay past the cache capacity: overflow flag")
    S, hid, B = 24, 512, 1
    L = Layer(hid, 4, 2, 1024, batch=B, seq=S + 1, gamma_noise=True, seed=33)
    sh = L.shard(2, 1)
    kv = sh.kv_cache(B, S + 2)
    sh.prefill(ATTN, L.dev["x"][:, :S].contiguous(), kv)
    xbuf = L.dev["x"][:, S].contiguous()
    pa = nan_like((B, hid))
    sh.decode(ATTN, xbuf, kv, out=pa)              # eager: length S + 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sh.decode(ATTN, xbuf, kv, out=pa)
    torch.cuda.synchronize()
    assert kv.length == S + 1                      # capture executes nothing
    g.replay()                                     # length S + 2: the capacity
    torch.cuda.synchronize()
    assert kv.length == S + 2
    g.replay()                                     # full: nothing appended, flag raised
    torch.cuda.synchronize()
    with pytest.raises(TPError) as e:
        _ = kv.length
    assert e.value.status == TP_E_KV_FULL
    assert bool(torch.isfinite(pa).all())
    with pytest.raises(TPError) as e:
        sh.decode(ATTN, xbuf, kv)
    assert e.value.status == TP_E_KV_FULL
    kv.length = S                                  # clears the flag
    assert kv.length == S
    del g


def test_decode_mlp_before_attn_is_refused():
    """A decode MLP stage on a shard that has run no ATTN stage returns
    TP_E_STATE before any launch."""
    from tensor_transformer_layer_tp_amd import TP_E_STATE
    announce("decode MLP before ATTN")
    L = Layer(512, 4, 4, 768, batch=1, seq=4, seed=16)
    sh = L.shard(2, 0)
    out = torch.full((1, 512), 3.0, device="cuda")
    with pytest.raises(TPError) as e:
        sh.decode(MLP, L.dev["x"][:, 0].contiguous(), out=out)
    assert e.value.status == TP_E_STATE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))


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
    spec = L.spec
    rows = [slice(r * n, (r + 1) * n) for r in range(tp)]
    x_rows = [L.exact["x"].reshape(T, hid)[rows[r]] for r in range(tp)]
    # each step against the oracle on the GPU's own inputs of that step
    n1_np = to_np(n1).reshape(T, hid)
    hs_np = [to_np(v) for v in hs]
    n2_np = to_np(n2).reshape(T, hid)
    for r in range(tp):
        assert_close(n1_np[rows[r]], O.norm1(x_rows[r], L.W, spec), f"n1 rows r{r}", "bf16")
    refa = [O.attn_from_n1(n1_np.reshape(B, S, hid), L.W, spec, tp, r) for r in range(tp)]
    for r in range(tp):
        assert_close(to_np(pa[r]), refa[r]["partial"], f"attn partial r{r}", "bf16")
    for r in range(tp):
        assert_close(hs_np[r], sp.reduce_scatter([to_np(p) for p in pa], x_rows[r], spec, tp, r),
                     f"h rows r{r} (reduce-scatter of the GPU partials)", "bf16")
        assert_close(hs_np[r], sp.reduce_scatter([a["partial"] for a in refa], x_rows[r], spec, tp, r),
                     f"h rows r{r}", "bf16")
        assert_close(n2_np[rows[r]], O.norm2(hs_np[r], L.W, spec), f"n2 rows r{r}", "bf16")
    refm = [O.mlp_from_n2(n2_np.reshape(B, S, hid), L.W, spec, tp, r) for r in range(tp)]
    for r in range(tp):
        assert_close(to_np(pm[r]), refm[r]["partial"], f"mlp partial r{r}", "bf16")
        assert_close(to_np(ys[r]), sp.reduce_scatter([m["partial"] for m in refm], hs_np[r], spec, tp, r),
                     f"y rows r{r} (chained)", "bf16")
    # end to end against the oracle's own sequence-parallel chain
    ref = sp.layer_sp(L.exact["x"], L.W, spec, tp)
    y = np.concatenate([to_np(v) for v in ys])
    rel, _ = report(y, np.concatenate(ref["y"]), f"sequence-parallel y end to end, t={tp}")
    assert rel <= 1e-2, f"sequence-parallel y: norm-relative error {rel:.3g}"
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


def test_70b_t8_prefill_reduce_equals_two_calls(layer70b):
    """The headline step's stages at their real shape (rank 0 of t=8, B=4,
    S=4096: eight rounds of 256x256 tiles, the twelve-wave sum epilogue):
    tp_shard_forward_prefill_reduce bit for bit against
    tp_shard_forward_prefill followed by tp_partial_reduce with the same seven
    other-rank partials, for h and y, and the caches."""
    announce("70B-shaped t=8 prefill with the reduce folded in, B=4 S=4096, against prefill + reduce")
    L = layer70b
    B, S, hid, tp = 4, 4096, 8192, 8
    sh_a, sh_b = L.shard(tp, 0), L.shard(tp, 0)
    kv_a, kv_b = sh_a.kv_cache(B, S), sh_b.kv_cache(B, S)
    x = L.dev["x"]
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    oth = [None] + [torch.randn((B, S, hid), generator=g, device="cuda") for _ in range(tp - 1)]
    pa = sh_a.prefill(ATTN, x, kv_a)
    h_ref = partial_reduce([pa] + oth[1:], residual=x)
    del pa
    h = sh_b.prefill_reduce(ATTN, x, oth, residual=x, kv=kv_b)
    torch.cuda.synchronize()
    assert torch.equal(h, h_ref), "h differs from prefill + partial_reduce"
    ka, va = kv_a.read()
    kb, vb = kv_b.read()
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    del ka, va, kb, vb
    pm = sh_a.prefill(MLP, h_ref)
    y_ref = partial_reduce([pm] + oth[1:], residual=h_ref)
    del pm
    y = sh_b.prefill_reduce(MLP, h, oth, residual=h)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "y differs from prefill + partial_reduce"
    assert torch.isfinite(y.float()).all()


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
    n_cfg = 19
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


@pytest.mark.parametrize("cfgs", [(14, 16), (15, 11), (12, 1)])
@pytest.mark.parametrize("cols0", [192, 448])
def test_forced_column_split_every_epilogue(cfgs, cols0):
    """Every epilogue -- the rotary Q/K/V scatter, SwiGLU, GELU and the fp32
    partial -- run as two launches over column ranges, the second starting
    at column cols0 (448 splits a Q head between the launches), against the
    oracle.  The planner takes such splits on its own only for a few shapes
    (the 70B t=8 Q/K/V projection, the 7B gate/up at 2048 unsharded or 8192
    sharded tokens); this reaches each epilogue's column offset."""
    from tensor_transformer_layer_tp_amd import gemm_plan, set_gemm_split
    announce(f"forced two-launch column split at {cols0}, configurations {cfgs}")
    t, r, S = 2, 1, 300
    Ls = Layer(1024, 8, 4, 2816, batch=1, seq=S, gamma_noise=True, seed=17)
    Lg = Layer(1024, 8, 4, 2816, swiglu=False, rope=False, batch=1, seq=S, gamma_noise=True, seed=18)
    h = synth.to_storage(synth.draw_normal((1, S, 1024), 19), "bf16")
    try:
        set_gemm_split(cfgs[0], cfgs[1], cols0)
        assert [c for _, c in gemm_plan(S, 2816, 1024, "swiglu")] == [cols0, 2816 - cols0]
        assert [c for _, c in gemm_plan(S, 1024, 1024, "qkv")] == [cols0, 1024 - cols0]
        for L, name in ((Ls, "swiglu"), (Lg, "gelu")):
            sh = L.shard(t, r)
            pa = sh.prefill(ATTN, L.dev["x"], out=nan_like((1, S, 1024)))
            o = sh.debug_tensor("o", (S, 512))
            pm = sh.prefill(MLP, h.cuda(), out=nan_like((1, S, 1024)))
            act = sh.debug_tensor("act", (S, 1408))
            torch.cuda.synchronize()
            ref_a = O.attn_stage(L.exact["x"], L.W, L.spec, t, r)
            ref_m = O.mlp_stage(h.float().numpy(), L.W, L.spec, t, r)
            assert_close(to_np(o), ref_a["o"].transpose(0, 2, 1, 3).reshape(S, 512), f"{name}: attention o", "bf16")
            assert_close(to_np(pa), ref_a["partial"], f"{name}: attn partial", "bf16")
            assert_close(to_np(act), ref_m["act"].reshape(S, 1408), f"{name}: act", "bf16")
            assert_close(to_np(pm), ref_m["partial"], f"{name}: mlp partial", "bf16")
    finally:
        set_gemm_split(0, 0, 0)


# ---------------------------------------------------------------- crossover sweep shapes (7B, t=2 and t=1)

def test_sweep_7b_t1_b1_s2048_full():
    """The unsharded 7B layer (t = 1: 32 heads, Q/K/V N 12288, SwiGLU 11008)
    at B=1, S=2048, every element of every tensor.  Its gate/up projection
    runs as the planner's two-launch column split (16384 + 5632 columns)."""
    from tensor_transformer_layer_tp_amd import gemm_plan
    announce("7B-shaped t=1 prefill B=1 S=2048 (crossover sweep), full compare")
    assert [c for _, c in gemm_plan(2048, 22016, 4096, "swiglu")] == [16384, 5632]
    L = Layer(4096, 32, 32, 11008, batch=1, seq=2048, seed=0)
    run_chain(L, 1, 1, 2048)


@pytest.mark.parametrize("tp", [2, 1])
def test_sweep_7b_b4_s512_full(tp):
    """A batched crossover point, B=4 x S=512, sharded (both ranks) and
    unsharded, every element (t = 1 takes the gate/up column split)."""
    announce(f"7B-shaped t={tp} prefill B=4 S=512 (crossover sweep), full compare")
    L = Layer(4096, 32, 32, 11008, batch=4, seq=512, seed=0)
    run_chain(L, tp, 4, 512)


def test_sweep_7b_t2_b4_s2048_sampled():
    """The sharded 7B layer at B=4, S=2048 (8192 tokens: the gate/up
    projection runs as the planner's 10240 + 768 column split), both ranks
    and both reduces, checked on sampled rows of sequences 0 and 3 and on
    their whole K/V cache."""
    from tensor_transformer_layer_tp_amd import gemm_plan
    announce("7B-shaped t=2 prefill B=4 S=2048 (crossover sweep), sampled rows")
    assert [c for _, c in gemm_plan(8192, 11008, 4096, "swiglu")] == [10240, 768]
    L = Layer(4096, 32, 32, 11008, batch=4, seq=2048, seed=0)
    sampled_chain({k: v for k, v in L.dev.items() if k != "x"}, L.W, L.spec, 2, L.dev["x"],
                  {0: L.exact["x"][0], 3: L.exact["x"][3]}, sample_rows(2048, 7))


def test_sweep_7b_t1_b64_s8192_sampled():
    """The largest crossover point: the unsharded 7B layer at B=64, S=8192
    (524 288 tokens: activations, the cache, act and the fp32 partials all
    pass 2^31 elements, so the 64-bit offsets are exercised end to end).
    Sequences 0 and 63 hold seeded NumPy inputs and are checked on sampled
    rows (first, last and 62 random) and on their whole K/V cache; the other
    sequences hold device-drawn filler, which attention never mixes in."""
    announce("7B-shaped t=1 prefill B=64 S=8192 (largest crossover point), sampled rows")
    B, S, hid = 64, 8192, 4096
    L = Layer(hid, 32, 32, 11008, seq=0, seed=0)
    x_dev = synth.draw_normal_device((B, S, hid), 5)
    x_np = {}
    for b, seed in ((0, 81), (B - 1, 82)):
        st = synth.to_storage(synth.draw_normal((S, hid), seed), "bf16")
        x_np[b] = st.float().numpy()
        x_dev[b].copy_(st.cuda())
    sampled_chain({k: v for k, v in L.dev.items()}, L.W, L.spec, 1, x_dev, x_np, sample_rows(S, 8))
    del x_dev
    torch.cuda.empty_cache()
