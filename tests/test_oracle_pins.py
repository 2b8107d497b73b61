"""Pins for the CPU oracle: it is checked against things other than itself.

- closed forms and special cases of attention, RoPE and RMSNorm;
- PyTorch CPU float64 library routines for the textbook pieces;
- an independent brute-force scalar implementation on tiny layers;
- the tensor-parallel identities the pages state (column-parallel outputs
  concatenate to the full projection; row-parallel partials sum to the full
  output; the output projection still needs the reduce);
- the partition rules (tests/golden/partition_cases.txt, with citations);
- decode at position L equals row L of a prefill over L+1 tokens;
- planted mistakes in the oracle must fail these pins.
"""

import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute, layer as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def weights(spec: O.Spec, seed=1, gamma_noise=True):
    d = spec.head_dim
    h, H, Hk, Fw = spec.hidden, spec.heads, spec.kv_heads, spec.ffn
    W = {
        "wq": rnd((H * d, h), seed + 1, 0.3),
        "wk": rnd((Hk * d, h), seed + 2, 0.3),
        "wv": rnd((Hk * d, h), seed + 3, 0.3),
        "wo": rnd((h, H * d), seed + 4, 0.3),
        "w_up": rnd((Fw, h), seed + 6, 0.3),
        "w_down": rnd((h, Fw), seed + 7, 0.3),
        "g1": 1 + (rnd((h,), seed + 8, 0.1) if gamma_noise else 0),
        "g2": 1 + (rnd((h,), seed + 9, 0.1) if gamma_noise else 0),
    }
    if spec.swiglu:
        W["w_gate"] = rnd((Fw, h), seed + 5, 0.3)
    return W


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_hand_cases():
    one = 1.0
    cases = [
        (0.0, 0.0),
        (one, one),
        (one + 2**-8, one),                       # tie -> even (1.0)
        (one + 3 * 2**-8, one + 2**-6),           # tie -> even mantissa
        (one + 2**-8 + 2**-30, one + 2**-7),      # just above the tie
        (-(one + 2**-8 + 2**-30), -(one + 2**-7)),
        (3.0 * 2**100, 3.0 * 2**100),
        (2**-133, 2**-133),                       # smallest bf16 subnormal
        (1.5 * 2**-133, 2 * 2**-133),             # subnormal tie -> even
        (0.4 * 2**-133, 0.0),
        (255.5, 256.0),                           # 255.5: spacing 1 at [128,256) -> tie -> 256 (even)
        (254.5, 254.0),                           # tie -> 254 (even)
    ]
    for a, want in cases:
        assert O.bf16_round(np.float64(a)) == want, a


def test_bf16_round_matches_torch_conversion():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32)
    x = np.concatenate([x, x * 1e-30, x * 1e30, (x * 1e-39).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- elementwise pieces

def test_rmsnorm_matches_torch():
    x = rnd((3, 7, 64), 2)
    g = 1 + rnd((64,), 3, 0.1)
    want = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, g, 1e-5), want, rtol=1e-13, atol=1e-13)


def test_rmsnorm_scale_invariant():
    x = rnd((4, 32), 4)
    g = 1 + rnd((32,), 5, 0.1)
    np.testing.assert_allclose(O.rmsnorm(7.5 * x, g, 0.0), O.rmsnorm(x, g, 0.0), rtol=1e-13)
    # unit RMS rows with gamma = 1 are fixed points when eps = 0
    u = x / np.sqrt((x * x).mean(-1, keepdims=True))
    np.testing.assert_allclose(O.rmsnorm(u, np.ones(32), 0.0), u, rtol=1e-13)


def test_activations_match_torch():
    z = np.linspace(-12, 12, 2001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_erf(z), F.gelu(torch.from_numpy(z), approximate="none").numpy(),
                               rtol=1e-14, atol=1e-15)
    assert O.gelu_erf(0.0) == 0.0 and abs(O.gelu_erf(40.0) - 40.0) < 1e-12 and abs(O.gelu_erf(-40.0)) < 1e-12
    assert O.silu(0.0) == 0.0


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    u = rnd((2, 3, 5, 16), 6)
    np.testing.assert_array_equal(O.rope(u, np.zeros(5), 1e4), u)


def test_rope_is_complex_rotation():
    # rotate-half RoPE == multiply z_i = u_i + i*u_{i+d/2} by exp(i * p * base^(-2i/d))
    d, S = 16, 9
    u = rnd((S, d), 7)
    pos = np.arange(S) * 3 + 5
    z = u[:, : d // 2] + 1j * u[:, d // 2:]
    w = np.exp(1j * pos[:, None] * 500.0 ** (-np.arange(d // 2) * 2.0 / d)[None, :])
    zr = z * w
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(O.rope(u, pos, 500.0), want, rtol=1e-12, atol=1e-12)


def test_rope_preserves_norm_and_relative_positions():
    d = 32
    q, k = rnd((1, d), 8), rnd((1, d), 9)
    for p, l, c in [(5, 2, 11), (100, 3, 1000), (7, 7, 3)]:
        qp, kl = O.rope(q, [p], 1e4), O.rope(k, [l], 1e4)
        qc, kc = O.rope(q, [p + c], 1e4), O.rope(k, [l + c], 1e4)
        assert abs(np.sum(qp * kl) - np.sum(qc * kc)) < 1e-11
        assert abs(np.linalg.norm(qp) - np.linalg.norm(q)) < 1e-12


# ---------------------------------------------------------------- attention

def test_attention_matches_torch_sdpa_gqa():
    B, H, Hk, S, d = 2, 6, 2, 11, 8
    q, k, v = rnd((B, H, S, d), 10), rnd((B, Hk, S, d), 11), rnd((B, Hk, S, d), 12)
    pos = np.arange(S)
    got = O.attention(q, k, v, pos, pos)
    kr = torch.from_numpy(k).repeat_interleave(H // Hk, dim=1)
    vr = torch.from_numpy(v).repeat_interleave(H // Hk, dim=1)
    want = F.scaled_dot_product_attention(torch.from_numpy(q), kr, vr, is_causal=True).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    d = 8
    # one position: output equals v
    q, k, v = rnd((1, 2, 1, d), 13), rnd((1, 1, 1, d), 14), rnd((1, 1, 1, d), 15)
    o = O.attention(q, k, v, [0], [0])
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(o[0, 1, 0], v[0, 0, 0], rtol=1e-14)
    # identical keys: uniform weights over the visible prefix
    S = 6
    q = rnd((1, 1, S, d), 16)
    k = np.broadcast_to(rnd((1, 1, 1, d), 17), (1, 1, S, d)).copy()
    v = rnd((1, 1, S, d), 18)
    o = O.attention(q, k, v, np.arange(S), np.arange(S))
    for i in range(S):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, : i + 1].mean(0), rtol=1e-12, atol=1e-14)


def test_attention_is_causal():
    B, H, S, d = 1, 2, 9, 8
    q, k, v = rnd((B, H, S, d), 19), rnd((B, H, S, d), 20), rnd((B, H, S, d), 21)
    pos = np.arange(S)
    base = O.attention(q, k, v, pos, pos)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:] += 3.0
    v2[:, :, 5:] -= 2.0
    pert = O.attention(q, k2, v2, pos, pos)
    np.testing.assert_array_equal(pert[:, :, :5], base[:, :, :5])
    assert np.abs(pert[:, :, 5:] - base[:, :, 5:]).max() > 1e-3


# ---------------------------------------------------------------- brute force

TINY = [
    O.Spec(16, 4, 4, 24, swiglu=True, mirror_bf16=False),
    O.Spec(16, 4, 2, 24, swiglu=True, mirror_bf16=False),          # GQA
    O.Spec(16, 4, 1, 8, swiglu=True, mirror_bf16=False),           # one KV head
    O.Spec(16, 2, 2, 12, swiglu=False, norm=False, rope=False, mirror_bf16=False),
    O.Spec(12, 2, 1, 10, swiglu=False, norm=True, rope=True, mirror_bf16=False),
    O.Spec(16, 4, 2, 24, swiglu=True, mirror_bf16=True),           # bf16 storage points
    O.Spec(16, 2, 2, 12, swiglu=False, norm=False, rope=False, mirror_bf16=True),
]


def _to_list(a):
    return np.asarray(a).tolist()


@pytest.mark.parametrize("spec", TINY, ids=lambda s: f"h{s.hidden}H{s.heads}k{s.kv_heads}F{s.ffn}"
                         f"{'sw' if s.swiglu else 'ge'}{'n' if s.norm else ''}{'r' if s.rope else ''}"
                         f"{'bf' if s.mirror_bf16 else ''}")
def test_layer_matches_brute_force(spec):
    B, S = 2, 5
    W = weights(spec, seed=31)
    x = rnd((B, S, spec.hidden), 32)
    if spec.mirror_bf16:
        x = O.bf16_round(x)
        W = {k: (O.bf16_round(v) if k not in ("g1", "g2") else v) for k, v in W.items()}
    want = brute.layer(_to_list(x), {k: _to_list(v) for k, v in W.items()},
                       hidden=spec.hidden, heads=spec.heads, kv_heads=spec.kv_heads, ffn=spec.ffn,
                       swiglu=spec.swiglu, norm=spec.norm, rope=spec.rope, eps=spec.eps,
                       theta=spec.rope_theta, mirror=spec.mirror_bf16)
    got = O.layer(x, W, spec, t=1)
    if spec.mirror_bf16:
        # both sides round at the same points; float64 summation order can
        # move a value across a rounding boundary, by one bf16 step at most
        np.testing.assert_allclose(got["h"], want["h"], rtol=2**-7, atol=1e-6)
        np.testing.assert_allclose(got["y"], want["y"], rtol=2**-6, atol=2**-6)
        frac_exact = np.mean(np.asarray(got["y"]) == np.asarray(want["y"]))
        assert frac_exact > 0.9
    else:
        np.testing.assert_allclose(got["h"], want["h"], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(got["y"], want["y"], rtol=1e-11, atol=1e-11)


def test_mirror_rounds_at_storage_points():
    spec = O.Spec(32, 4, 2, 64, mirror_bf16=True)
    W = weights(spec, seed=41)
    x = O.bf16_round(rnd((1, 6, 32), 42))
    out = O.layer(x, W, spec, t=2)
    for key in ("n1", "q", "k", "v", "o"):
        a = out["attn"][1][key]
        np.testing.assert_array_equal(O.bf16_round(a), a)
    for key in ("n2", "act"):
        a = out["mlp"][0][key]
        np.testing.assert_array_equal(O.bf16_round(a), a)
    np.testing.assert_array_equal(O.bf16_round(out["h"]), out["h"])
    np.testing.assert_array_equal(O.bf16_round(out["y"]), out["y"])
    # partials stay in high precision
    assert not np.array_equal(O.bf16_round(out["attn"][0]["partial"]), out["attn"][0]["partial"])


# ---------------------------------------------------------------- TP identities

@pytest.mark.parametrize("t", [1, 2, 4])
def test_column_parallel_concat_and_row_parallel_sum(t):
    spec = O.Spec(64, 8, 4, 96, mirror_bf16=False)
    W = weights(spec, seed=51)
    x = rnd((2, 7, 64), 52)
    full = O.layer(x, W, spec, t=1)
    shard = O.layer(x, W, spec, t=t)
    # column-parallel: the ranks' heads concatenate to the full q/k/v/o
    for key in ("q", "k", "v", "o"):
        cat = np.concatenate([a[key] for a in shard["attn"]], axis=1)
        np.testing.assert_allclose(cat, full["attn"][0][key], rtol=1e-12, atol=1e-12)
    cat = np.concatenate([m["act"] for m in shard["mlp"]], axis=-1)
    np.testing.assert_allclose(cat, full["mlp"][0]["act"], rtol=1e-12, atol=1e-12)
    # row-parallel: the partials sum to the full output
    s = sum(a["partial"] for a in shard["attn"])
    np.testing.assert_allclose(s, full["attn"][0]["partial"], rtol=1e-12, atol=1e-12)
    s = sum(m["partial"] for m in shard["mlp"])
    np.testing.assert_allclose(s, full["mlp"][0]["partial"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(shard["y"], full["y"], rtol=1e-12, atol=1e-12)


def test_single_partial_is_not_the_output():
    # the output projection still needs the reduce when t > 1
    spec = O.Spec(64, 8, 8, 96, mirror_bf16=False)
    W = weights(spec, seed=61)
    x = rnd((1, 5, 64), 62)
    full = O.layer(x, W, spec, t=1)
    shard = O.layer(x, W, spec, t=2)
    for r in range(2):
        assert np.abs(shard["attn"][r]["partial"] - full["attn"][0]["partial"]).max() > 1e-2
        assert np.abs(shard["mlp"][r]["partial"] - full["mlp"][0]["partial"]).max() > 1e-2


def test_head_permutation_across_ranks_keeps_output():
    # heads are independent: moving whole head blocks between ranks (with
    # their W_o columns) changes nothing once the partials are summed
    spec = O.Spec(64, 8, 8, 96, mirror_bf16=False)
    W = weights(spec, seed=71)
    x = rnd((1, 6, 64), 72)
    d = spec.head_dim
    perm = [4, 5, 6, 7, 0, 1, 2, 3]
    rows = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    W2 = dict(W, wq=W["wq"][rows], wk=W["wk"][rows], wv=W["wv"][rows], wo=W["wo"][:, rows])
    a = O.layer(x, W, spec, t=2)
    b = O.layer(x, W2, spec, t=2)
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["attn"][0]["partial"], b["attn"][1]["partial"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- partition rules

def _golden_partition_cases():
    cases = []
    with open(os.path.join(GOLDEN, "partition_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                H, Hk, Fw, t, expect = line.split()
                cases.append((int(H), int(Hk), int(Fw), int(t), expect))
    return cases


@pytest.mark.parametrize("case", _golden_partition_cases(), ids=str)
def test_partition_rules_golden(case):
    H, Hk, Fw, t, expect = case
    spec = O.Spec(H * 128, H, Hk, Fw)
    if expect == "ok":
        O.check_partition(spec, t)
        blocks = [O.rank_blocks(spec, t, r) for r in range(t)]
        assert sum(len(b[0]) for b in blocks) == H and sum(len(b[2]) for b in blocks) == Fw
    else:
        with pytest.raises(ValueError):
            O.check_partition(spec, t)


def test_rank_out_of_range():
    spec = O.Spec(64, 8, 8, 96)
    with pytest.raises(ValueError):
        O.check_partition(spec, 2, 2)
    with pytest.raises(ValueError):
        O.check_partition(spec, 2, -1)


# ---------------------------------------------------------------- prefill vs decode

@pytest.mark.parametrize("spec,t,r", [(O.Spec(64, 8, 2, 96, mirror_bf16=False), 2, 1),
                                      (O.Spec(64, 4, 4, 64, swiglu=False, norm=False, rope=False,
                                              mirror_bf16=False), 1, 0)])
def test_decode_equals_last_prefill_row(spec, t, r):
    W = weights(spec, seed=81)
    B, L = 2, 9
    x = rnd((B, L + 1, spec.hidden), 82)
    pre = O.attn_stage(x, W, spec, t, r)
    dec = O.decode_attn_stage(x[:, L], pre["k"][:, :, :L], pre["v"][:, :, :L], W, spec, t, r)
    np.testing.assert_allclose(dec["o"], pre["o"][:, :, L], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dec["partial"], pre["partial"][:, L], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dec["k_new"], pre["k"][:, :, L], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _brute_y(spec, x, W):
    return np.asarray(brute.layer(_to_list(x), {k: _to_list(v) for k, v in W.items()},
                                  hidden=spec.hidden, heads=spec.heads, kv_heads=spec.kv_heads,
                                  ffn=spec.ffn, swiglu=spec.swiglu, norm=spec.norm, rope=spec.rope,
                                  eps=spec.eps, theta=spec.rope_theta)["y"])


@pytest.mark.parametrize("mutation", ["rope_sign", "gqa_map", "drop_gamma", "wo_transposed",
                                      "swap_gate_up", "scale", "residual_twice"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    spec = O.Spec(16, 4, 2, 16, mirror_bf16=False)
    W = weights(spec, seed=91)
    x = rnd((1, 4, 16), 92)
    want = _brute_y(spec, x, W)
    if mutation == "rope_sign":
        orig = O.rope
        monkeypatch.setattr(O, "rope", lambda u, p, th: orig(u, -np.asarray(p), th))
    elif mutation == "gqa_map":
        def bad_attention(q, k, v, qp, kp):
            Hk = k.shape[1]
            idx = np.arange(q.shape[1]) % Hk          # interleaved instead of contiguous groups
            kk, vv = k[:, idx], v[:, idx]
            return O.__dict__["_orig_attention"](q, kk, vv, qp, kp)
        monkeypatch.setitem(O.__dict__, "_orig_attention", O.attention)
        monkeypatch.setattr(O, "attention", bad_attention)
    elif mutation == "drop_gamma":
        orig_rms = O.rmsnorm
        monkeypatch.setattr(O, "rmsnorm", lambda x_, g, e: orig_rms(x_, np.ones_like(g), e))
    elif mutation == "wo_transposed":
        W = dict(W, wo=np.ascontiguousarray(W["wo"].T))
    elif mutation == "swap_gate_up":
        W = dict(W, w_gate=W["w_up"], w_up=W["w_gate"])
    elif mutation == "scale":
        orig_att = O.attention
        monkeypatch.setattr(O, "attention", lambda q, k, v, a, b: orig_att(q * np.sqrt(q.shape[-1]), k, v, a, b))
    elif mutation == "residual_twice":
        orig_red = O.reduce
        monkeypatch.setattr(O, "reduce", lambda p, res, s: orig_red(list(p) + [res], res, s))
    # with t = 2 each rank of this layer holds one KV head, where any head
    # mapping is the same; the interleaved-group mistake shows at t = 1
    for t in ((1,) if mutation == "gqa_map" else (1, 2)):
        got = O.layer(x, W, spec, t=t)["y"]
        assert np.abs(got - want).max() > 1e-6, (mutation, t)


def test_row_restricted_stages_match_full_stages():
    spec = O.Spec(64, 8, 2, 96, mirror_bf16=True)
    W = weights(spec, seed=101)
    x = O.bf16_round(rnd((2, 13, 64), 102))
    rows = np.array([0, 5, 12])
    full = O.attn_stage(x, W, spec, 2, 1)
    part = O.attn_stage_rows(x, W, spec, 2, 1, rows)
    np.testing.assert_allclose(part["partial"], full["partial"][:, rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["o"], full["o"][:, :, rows], rtol=1e-12, atol=1e-12)
    m_full = O.mlp_stage(x, W, spec, 2, 0)
    m_part = O.mlp_stage_rows(x, W, spec, 2, 0, rows)
    np.testing.assert_allclose(m_part["partial"], m_full["partial"][:, rows], rtol=1e-12, atol=1e-12)
