"""Shared pieces of the GPU parity tests: seeded layers, device upload and
the tolerance checks.

Tolerances (written here once, used by every parity test):
- bf16 path: every element |gpu - oracle| <= 2e-2 + 1e-2 * |oracle|;
- fp32 path: max |gpu - oracle| <= 1e-5 * max |oracle| per tensor.
Every compared tensor uses these bounds on the result itself, the residual
sums h and y included.  The oracle mirrors the bf16 storage points (n1,
q/k/v, o, h, n2, act, y); partial sums are compared in fp32.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import layer as O
from tensor_transformer_layer_tp_amd import synth

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_REL = 1e-5


def assert_bf16_close(gpu, ref, name):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values (unwritten or overflow)"
    mag = np.abs(r)
    err = np.abs(g - r)
    bad = err > BF16_ATOL + BF16_RTOL * mag
    if bad.any():
        i = np.unravel_index(np.argmax(err - BF16_RTOL * mag), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; worst at {i}: "
                             f"gpu {g[i]} oracle {r[i]} (max abs err {err.max():.3g})")


def assert_f32_close(gpu, ref, name):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    scale = np.abs(r).max()
    err = np.abs(g - r).max()
    assert err <= F32_REL * scale, f"{name}: max abs err {err:.3g} > {F32_REL} * {scale:.3g}"


def assert_close(gpu, ref, name, dtype):
    if dtype == "bf16":
        assert_bf16_close(gpu, ref, name)
    else:
        assert_f32_close(gpu, ref, name)


def report(gpu, ref, name):
    """Diagnostic line (not an assertion): norm-relative error and the count
    of elements outside the bf16 bound."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    bad = int((err > BF16_ATOL + BF16_RTOL * np.abs(r)).sum())
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    print(f"[diag] {name}: norm-rel {rel:.3g}, max abs {err.max():.3g}, {bad} of {err.size} outside "
          f"{BF16_ATOL} + {BF16_RTOL}|ref|", flush=True)
    return rel, bad


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Layer:
    """A seeded layer: storage tensors on the device, exact values (float32
    arrays) for the oracle, and the oracle spec."""

    def __init__(self, hidden, heads, kv_heads, ffn, dtype="bf16", swiglu=True, norm=True, rope=True,
                 batch=1, seq=0, kv_len=0, decode_batch=1, seed=0, gamma_noise=False):
        raw = synth.draw_layer(hidden, heads, kv_heads, ffn, swiglu=swiglu, batch=batch, seq=seq,
                               kv_len=kv_len, decode_batch=decode_batch, seed=seed)
        if gamma_noise:
            raw["g1"] = 1 + synth.draw_normal((hidden,), seed + 1000, 0.1)
            raw["g2"] = 1 + synth.draw_normal((hidden,), seed + 1001, 0.1)
        self.dtype = dtype
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.spec = O.Spec(hidden, heads, kv_heads, ffn, swiglu=swiglu, norm=norm, rope=rope,
                           mirror_bf16=(dtype == "bf16"))
        self.dev = {}
        self.exact = {}
        for k, a in raw.items():
            st = synth.to_storage(a, dtype)
            self.exact[k] = st.float().numpy()           # exact stored values (float32 holds bf16 exactly)
            self.dev[k] = st.to("cuda")
        del raw
        self.W = {k: v for k, v in self.exact.items() if k not in ("x", "k_cache", "v_cache", "x_dec")}

    def shard(self, tp, rank):
        from tensor_transformer_layer_tp_amd import Shard
        s = self.spec
        sh = Shard(s.hidden, s.heads, s.kv_heads, s.ffn, tp, rank, dtype=self.dtype,
                   act="swiglu" if s.swiglu else "gelu", rmsnorm=s.norm, rope=s.rope)
        sh.load_weights({k: v for k, v in self.dev.items() if k not in ("x", "k_cache", "v_cache", "x_dec")})
        return sh


def rank_cache(full_cache: np.ndarray, spec, tp, rank) -> np.ndarray:
    """Rank r's KV heads of a full [B, Hkv, L, d] cache."""
    _, kb, _ = O.rank_blocks(spec, tp, rank)
    return full_cache[:, kb.start:kb.stop]
