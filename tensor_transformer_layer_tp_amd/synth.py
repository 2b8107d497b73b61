"""Seeded synthetic inputs shaped like LLaMA-class layers.

This module only draws random numbers and holds the workload table; it holds
none of the layer's arithmetic, so both the GPU path and the CPU oracle can
take their inputs from it.

Draw order for one layer (NumPy ``default_rng(seed)``, PCG64,
``standard_normal(dtype=float32)``): x, W_q, W_k, W_v, W_o, W_gate (the first
FFN matrix W_1 for a GELU FFN), W_up (SwiGLU only), W_down, then the KV-cache
fill (K then V, all KV heads), then the decode token.  Activations and the
cache fill are N(0, 1); weight matrices are 0.02 * N(0, 1).  RMSNorm gains
are 1.  For bf16 workloads every draw is rounded to bfloat16 (nearest, ties
to even) by torch's dtype conversion; both sides receive those exact values.
"""

from __future__ import annotations

import dataclasses

import numpy as np

WEIGHT_STD = np.float32(0.02)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    heads: int
    kv_heads: int
    ffn: int
    tp: int
    rank: int
    dtype: str            # "bf16" or "f32"
    swiglu: bool = True
    norm: bool = True
    rope: bool = True
    batch: int = 1
    seq: int = 0          # prefill prompt length (0: none)
    kv_len: int = 0       # decode: cache length before the new token (0: none)
    decode_batch: int = 1


# The layer shapes the measurements use: a tiny fp32 layer, a 7B-shaped
# (hidden 4096, 32 heads, FFN 11008) and a 70B-shaped GQA layer (hidden 8192,
# 64 query / 8 KV heads, FFN 28672), each as one rank of a t-way split.
WORKLOADS = {
    "tiny-f32-t2": Workload("tiny-f32-t2", 256, 4, 4, 1024, 2, 0, "f32",
                            swiglu=False, norm=False, rope=False, batch=1, seq=32),
    "7b-t2-prefill": Workload("7b-t2-prefill", 4096, 32, 32, 11008, 2, 0, "bf16",
                              batch=1, seq=2048),
    "7b-t4-decode": Workload("7b-t4-decode", 4096, 32, 32, 11008, 4, 0, "bf16",
                             kv_len=1024, decode_batch=1),
    "70b-t8-prefill": Workload("70b-t8-prefill", 8192, 64, 8, 28672, 8, 0, "bf16",
                               batch=4, seq=4096),
    "70b-t8-decode": Workload("70b-t8-decode", 8192, 64, 8, 28672, 8, 0, "bf16",
                              kv_len=4096, decode_batch=1),
}

# batch x prompt-length grid of the 7B crossover sweep (t = 2 shard vs t = 1)
SWEEP_BATCH = (1, 4, 16, 64)
SWEEP_SEQ = (128, 512, 2048, 8192)


def draw_layer(hidden, heads, kv_heads, ffn, *, swiglu=True, batch=1, seq=0,
               kv_len=0, decode_batch=1, seed=0):
    """Return a dict of float32 NumPy arrays in the fixed draw order.

    Keys: x [batch, seq, hidden] (absent if seq == 0), wq, wk, wv, wo,
    w_gate (SwiGLU only), w_up, w_down, g1, g2, and when kv_len > 0:
    k_cache, v_cache [decode_batch, kv_heads, kv_len, d] and x_dec
    [decode_batch, hidden].  For a GELU FFN the first FFN matrix is
    returned as w_up (it is drawn in W_gate's slot)."""
    d = hidden // heads
    rng = np.random.default_rng(seed)
    n = rng.standard_normal
    out = {}
    if seq > 0:
        out["x"] = n((batch, seq, hidden), dtype=np.float32)
    out["wq"] = n((heads * d, hidden), dtype=np.float32) * WEIGHT_STD
    out["wk"] = n((kv_heads * d, hidden), dtype=np.float32) * WEIGHT_STD
    out["wv"] = n((kv_heads * d, hidden), dtype=np.float32) * WEIGHT_STD
    out["wo"] = n((hidden, heads * d), dtype=np.float32) * WEIGHT_STD
    first = n((ffn, hidden), dtype=np.float32) * WEIGHT_STD
    if swiglu:
        out["w_gate"] = first
        out["w_up"] = n((ffn, hidden), dtype=np.float32) * WEIGHT_STD
    else:
        out["w_up"] = first
    out["w_down"] = n((hidden, ffn), dtype=np.float32) * WEIGHT_STD
    out["g1"] = np.ones(hidden, np.float32)
    out["g2"] = np.ones(hidden, np.float32)
    if kv_len > 0:
        out["k_cache"] = n((decode_batch, kv_heads, kv_len, d), dtype=np.float32)
        out["v_cache"] = n((decode_batch, kv_heads, kv_len, d), dtype=np.float32)
        out["x_dec"] = n((decode_batch, hidden), dtype=np.float32)
    return out


def draw_workload(w: Workload, seed=0, batch=None, seq=None):
    return draw_layer(w.hidden, w.heads, w.kv_heads, w.ffn, swiglu=w.swiglu,
                      batch=w.batch if batch is None else batch,
                      seq=w.seq if seq is None else seq, kv_len=w.kv_len,
                      decode_batch=w.decode_batch, seed=seed)


def draw_normal(shape, seed, scale=1.0):
    """An extra seeded N(0, scale^2) float32 array (e.g. a synthetic h)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)


def to_storage(a, dtype: str):
    """float32 array -> torch CPU tensor of the storage type ("bf16" rounds
    to nearest even via torch's conversion; "f32" is a copy)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def as_f64(t) -> np.ndarray:
    """The exact values of a torch storage tensor as a float64 array."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def draw_layer_device(hidden, heads, kv_heads, ffn, *, seed=0, device="cuda", dtype=None):
    """Timing-only variant of ``draw_layer``: the same matrices, scales and
    order, drawn on the device with torch's generator (Philox) and cast to
    the storage type, for layers too large to draw quickly on the host.  The
    values differ from the NumPy draws, so these inputs are never compared
    with the oracle.  Returns the weight dict (wq, wk, wv, wo, w_gate, w_up,
    w_down, g1, g2) of a SwiGLU layer."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d = hidden // heads

    def n(shape, scale):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale).to(dtype)

    std = float(WEIGHT_STD)
    return {
        "wq": n((heads * d, hidden), std), "wk": n((kv_heads * d, hidden), std),
        "wv": n((kv_heads * d, hidden), std), "wo": n((hidden, heads * d), std),
        "w_gate": n((ffn, hidden), std), "w_up": n((ffn, hidden), std), "w_down": n((hidden, ffn), std),
        "g1": torch.ones(hidden, device=device, dtype=dtype), "g2": torch.ones(hidden, device=device, dtype=dtype),
    }


def draw_normal_device(shape, seed, scale=1.0, device="cuda", dtype=None):
    """N(0, scale^2) device tensor in the storage type (torch's generator):
    for timing, or as filler in rows that are never compared."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale
    return t.to(dtype or torch.bfloat16)
