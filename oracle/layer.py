"""Float64 oracle of a Megatron-style tensor-parallel transformer layer shard.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What the pages fix (cited by page title and section):

* undercodenews post 110319 on tensor parallelism in transformers, section
  "the Original":
  - attention builds Q, K and V as linear projections of the input, splits
    them into heads, attends per head independently and concatenates the
    heads;
  - the FFN is two linear layers with an activation between them;
  - a column-parallel linear multiplies the full input by a column slice of
    the weight, and the slices' outputs concatenate;
  - a row-parallel linear multiplies matching blocks and yields partial
    results that an all-reduce sums;
  - the Q/K/V projections are column-parallel, so every rank owns a subset
    of the heads and attends locally; the output projection is
    row-parallel; the FFN's first linear is column-parallel and its second
    row-parallel;
  - the TP degree may not exceed the head count, the head count must divide
    by it, and so must the FFN hidden width.
* netray glossary "What Is Tensor Parallelism?", section "Tensor Parallelism
  Explained": weight matrices are partitioned by rows or columns and the
  partial results are combined with an all-reduce.
* byteledger "Tensor Parallelism: Splitting One Layer Across GPUs", section
  "Interaction with the rest of serving": the KV cache is split across the
  devices too.
* clusterbid "When Tensor Parallelism Makes a Small Model Slower": decode is
  a sequence of one-token steps; prefill runs the same layer over a prompt.

Readings taken where the pages are silent (each is a choice, stated here so
that the code can be checked against it):

1. sequential pre-norm block: h = x + Attn(Norm1(x)), y = h + FFN(Norm2(h));
2. RMSNorm, n = x / sqrt(mean(x^2) + eps) * gamma, replicated on every rank
   (the column-parallel input is the full input); configurations without a
   norm use n = x;
3. rotate-half rotary embedding on q and k, pairs (i, i + d/2),
   theta_i = base^(-2i/d), prefill positions 0..S-1, decode position L;
4. scale 1/sqrt(d), causal mask key_pos <= query_pos;
5. grouped-query attention with contiguous groups: query head j reads KV
   head floor(j / (H / H_kv));
6. rank r owns contiguous blocks: query heads [r H/t, (r+1) H/t), KV heads
   [r H_kv/t, (r+1) H_kv/t), FFN columns [r F/t, (r+1) F/t);
7. SwiGLU act = SiLU(n W_gate^T) * (n W_up^T), or exact-erf GELU
   act = GELU(n W_1^T) for the two-matrix FFN; no biases anywhere;
8. the residual is added once, after the rank partials are summed in rank
   order;
9. bf16 configurations store bf16 at: n1, q/k/v after the rotary embedding,
   the attention output o, h, n2, act and y; partial sums stay in high
   precision.  ``mirror_bf16=True`` rounds at exactly those points (RNE);
   all arithmetic between them is float64.
"""

from __future__ import annotations

import dataclasses

import numpy as np
from scipy.special import erf


# --------------------------------------------------------------------------
# spec and partition rules


@dataclasses.dataclass(frozen=True)
class Spec:
    hidden: int
    heads: int
    kv_heads: int
    ffn: int
    swiglu: bool = True        # False: GELU(erf) two-matrix FFN
    norm: bool = True          # RMSNorm before attention and FFN
    rope: bool = True
    eps: float = 1e-5
    rope_theta: float = 10000.0
    mirror_bf16: bool = True   # round to bf16 at the storage points

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads


def check_partition(spec: Spec, t: int, r: int = 0) -> None:
    """Raise ValueError unless the layer splits t ways (undercodenews post
    110319, "the Original": degree <= heads, heads and FFN width divisible;
    the KV-head count must divide too for the KV heads to split)."""
    if t < 1:
        raise ValueError("tp degree must be >= 1")
    if spec.hidden % spec.heads:
        raise ValueError("hidden must divide by heads")
    if spec.heads % spec.kv_heads:
        raise ValueError("heads must divide by kv_heads")
    if t > spec.heads:
        raise ValueError("tp degree exceeds head count")
    if spec.heads % t or spec.kv_heads % t or spec.ffn % t:
        raise ValueError("heads, kv_heads and ffn must divide by the tp degree")
    if not 0 <= r < t:
        raise ValueError("rank out of range")


def rank_blocks(spec: Spec, t: int, r: int):
    """Contiguous blocks owned by rank r: (query heads, kv heads, ffn cols)."""
    check_partition(spec, t, r)
    hl, kl, fl = spec.heads // t, spec.kv_heads // t, spec.ffn // t
    return (range(r * hl, (r + 1) * hl), range(r * kl, (r + 1) * kl),
            range(r * fl, (r + 1) * fl))


# --------------------------------------------------------------------------
# elementwise pieces


def bf16_round(a) -> np.ndarray:
    """Nearest bfloat16 value of each float64 element, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range, so for
    |a| in [2^(e-1), 2^e) the spacing is 2^(e-8); below the smallest normal
    (2^-126) the spacing stays 2^-133.  Values beyond bf16's finite range
    are not expected here and are not saturated.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    return np.rint(a / q) * q


def _store(spec: Spec, a: np.ndarray) -> np.ndarray:
    return bf16_round(a) if spec.mirror_bf16 else np.asarray(a, np.float64)


def rmsnorm(x, gamma, eps):
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu_erf(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def rope(u, positions, theta):
    """Rotate-half rotary embedding of u [..., S, d] at the given positions
    [S]: the pair (u_i, u_{i+d/2}) turns by angle pos * theta^(-2i/d)."""
    u = np.asarray(u, np.float64)
    d = u.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]   # [S, d/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q, k, v, q_pos, k_pos):
    """Softmax attention, one head at a time.

    q [B, Hq, Sq, d], k/v [B, Hk, Sk, d]; query head j reads KV head
    floor(j / (Hq / Hk)).  A key is visible to a query when its position is
    not after the query's.  Returns o [B, Hq, Sq, d].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Sq, d = q.shape
    Hk = k.shape[1]
    group = Hq // Hk
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]   # [Sq, Sk]
    o = np.empty_like(q)
    for b in range(B):
        for j in range(Hq):
            g = j // group
            s = (q[b, j] @ k[b, g].T) / np.sqrt(d)
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            o[b, j] = p @ v[b, g]
    return o


# --------------------------------------------------------------------------
# the two stages of a rank's shard


def _heads_rows(block: range, d: int) -> slice:
    return slice(block.start * d, block.stop * d)


def qkv_rank(n1, W, spec: Spec, t: int, r: int, positions):
    """Column-parallel Q/K/V projection of rank r (its own heads), rotary
    embedding at ``positions``, stored at bf16 when mirroring.

    n1 [B, S, hidden] -> q [B, H_l, S, d], k/v [B, Hkv_l, S, d]."""
    hb, kb, _ = rank_blocks(spec, t, r)
    d = spec.head_dim
    B, S, _ = n1.shape
    q = n1 @ np.asarray(W["wq"], np.float64)[_heads_rows(hb, d)].T
    k = n1 @ np.asarray(W["wk"], np.float64)[_heads_rows(kb, d)].T
    v = n1 @ np.asarray(W["wv"], np.float64)[_heads_rows(kb, d)].T
    q = q.reshape(B, S, len(hb), d).transpose(0, 2, 1, 3)
    k = k.reshape(B, S, len(kb), d).transpose(0, 2, 1, 3)
    v = v.reshape(B, S, len(kb), d).transpose(0, 2, 1, 3)
    if spec.rope:
        q = rope(q, positions, spec.rope_theta)
        k = rope(k, positions, spec.rope_theta)
    return _store(spec, q), _store(spec, k), _store(spec, v)


def norm1(x, W, spec: Spec):
    if not spec.norm:
        return np.asarray(x, np.float64)
    return _store(spec, rmsnorm(x, W["g1"], spec.eps))


def norm2(h, W, spec: Spec):
    if not spec.norm:
        return np.asarray(h, np.float64)
    return _store(spec, rmsnorm(h, W["g2"], spec.eps))


def out_proj_rank(o, W, spec: Spec, t: int, r: int):
    """Row-parallel output projection: rank r multiplies its heads' columns
    of W_o by its own attention output.  o [B, H_l, S, d] -> partial
    [B, S, hidden] (one summand of the all-reduce)."""
    hb, _, _ = rank_blocks(spec, t, r)
    d = spec.head_dim
    B, Hl, S, _ = o.shape
    o_tok = o.transpose(0, 2, 1, 3).reshape(B, S, Hl * d)
    return o_tok @ np.asarray(W["wo"], np.float64)[:, _heads_rows(hb, d)].T


def attn_stage(x, W, spec: Spec, t: int = 1, r: int = 0):
    """Prefill ATTN stage of rank r over x [B, S, hidden]: norm, own-head
    Q/K/V, causal attention over positions 0..S-1, row-parallel partial."""
    x = np.asarray(x, np.float64)
    return attn_from_n1(norm1(x, W, spec), W, spec, t, r)


def attn_from_n1(n1, W, spec: Spec, t: int = 1, r: int = 0):
    """The ATTN stage after its norm: n1 [B, S, hidden] is the normalised
    stage input (computed by this rank, or gathered from the ranks'
    sequence shards)."""
    n1 = np.asarray(n1, np.float64)
    S = n1.shape[1]
    pos = np.arange(S)
    q, k, v = qkv_rank(n1, W, spec, t, r, pos)
    o = _store(spec, attention(q, k, v, pos, pos))
    partial = out_proj_rank(o, W, spec, t, r)
    return {"n1": n1, "q": q, "k": k, "v": v, "o": o, "partial": partial}


def mlp_stage(h, W, spec: Spec, t: int = 1, r: int = 0):
    """FFN stage of rank r over the reduced h [B, S, hidden]: norm, the
    column-parallel up (and gate) projection of the rank's FFN columns with
    the activation, then the row-parallel down projection's partial."""
    h = np.asarray(h, np.float64)
    return mlp_from_n2(norm2(h, W, spec), W, spec, t, r)


def mlp_from_n2(n2, W, spec: Spec, t: int = 1, r: int = 0):
    """The FFN stage after its norm: n2 [B, S, hidden] is the normalised
    stage input."""
    n2 = np.asarray(n2, np.float64)
    _, _, fb = rank_blocks(spec, t, r)
    cols = slice(fb.start, fb.stop)
    if spec.swiglu:
        g = n2 @ np.asarray(W["w_gate"], np.float64)[cols].T
        u = n2 @ np.asarray(W["w_up"], np.float64)[cols].T
        act = silu(g) * u
    else:
        act = gelu_erf(n2 @ np.asarray(W["w_up"], np.float64)[cols].T)
    act = _store(spec, act)
    partial = act @ np.asarray(W["w_down"], np.float64)[:, cols].T
    return {"n2": n2, "act": act, "partial": partial}


def reduce(partials, residual, spec: Spec):
    """The all-reduce's sum, done once: residual + sum of rank partials in
    rank order, stored at bf16 when mirroring."""
    s = np.zeros_like(np.asarray(partials[0], np.float64))
    for p in partials:
        s = s + np.asarray(p, np.float64)
    return _store(spec, s + np.asarray(residual, np.float64))


def layer(x, W, spec: Spec, t: int = 1):
    """Whole layer as t ranks would compute it: every rank's stages, the
    two reduces.  With t = 1 this is the unsharded layer."""
    attn = [attn_stage(x, W, spec, t, r) for r in range(t)]
    h = reduce([a["partial"] for a in attn], x, spec)
    mlp = [mlp_stage(h, W, spec, t, r) for r in range(t)]
    y = reduce([m["partial"] for m in mlp], h, spec)
    return {"attn": attn, "h": h, "mlp": mlp, "y": y}


# --------------------------------------------------------------------------
# decode: one new token per sequence against the rank's KV cache


def decode_attn_stage(x_new, k_cache, v_cache, W, spec: Spec, t: int = 1, r: int = 0):
    """Decode ATTN stage of rank r.

    x_new [B, hidden] is the token at position L = k_cache.shape[2];
    k_cache/v_cache [B, Hkv_l, L, d] hold rank r's KV heads (already
    rotated).  The new k, v are appended at slot L and the query attends to
    positions 0..L.  Returns the new cache rows, o and the partial [B, hidden].
    """
    x_new = np.asarray(x_new, np.float64)
    B = x_new.shape[0]
    L = k_cache.shape[2]
    n1 = norm1(x_new[:, None, :], W, spec)
    q, k, v = qkv_rank(n1, W, spec, t, r, np.array([L]))
    K = np.concatenate([np.asarray(k_cache, np.float64), k], axis=2)
    V = np.concatenate([np.asarray(v_cache, np.float64), v], axis=2)
    o = _store(spec, attention(q, K, V, np.array([L]), np.arange(L + 1)))
    partial = out_proj_rank(o, W, spec, t, r)[:, 0, :]
    return {"n1": n1[:, 0, :], "q": q[:, :, 0, :], "k_new": k[:, :, 0, :],
            "v_new": v[:, :, 0, :], "o": o[:, :, 0, :], "partial": partial}


def attn_stage_rows(x, W, spec: Spec, t: int, r: int, rows):
    """The prefill ATTN stage of rank r evaluated only at the token rows
    ``rows`` (indices into the sequence) of every batch element: the same
    definition as ``attn_stage``, restricted so that large layers stay
    checkable.  Row i needs the keys and values of tokens 0..i, so those are
    computed for the prefix up to the largest requested row.

    Returns {"o": [B, H_l, len(rows), d], "partial": [B, len(rows), hidden],
    "k", "v": [B, Hkv_l, max(rows)+1, d]}."""
    x = np.asarray(x, np.float64)
    rows = np.asarray(rows)
    last = int(rows.max()) + 1
    pos = np.arange(last)
    n1 = norm1(x[:, :last], W, spec)
    _, k, v = qkv_rank(n1, W, spec, t, r, pos)
    q, _, _ = qkv_rank(n1[:, rows], W, spec, t, r, rows)
    o = _store(spec, attention(q, k, v, rows, pos))
    partial = out_proj_rank(o, W, spec, t, r)
    return {"o": o, "partial": partial, "k": k, "v": v}


def mlp_stage_rows(h, W, spec: Spec, t: int, r: int, rows):
    """The MLP stage of rank r at the token rows ``rows`` only (rows are
    independent in this stage)."""
    return mlp_stage(np.asarray(h)[:, rows], W, spec, t, r)
