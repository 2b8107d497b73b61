"""Brute-force scalar oracle for tiny layers (pure Python loops, math module).

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.layer`` (no
shared helpers) so that a slip in one -- a dropped term, a swapped operand,
a wrong head-to-KV-head mapping, a rounding point in the wrong place -- shows
up as a mismatch.  It computes the *unsharded* layer only: one token at a
time, one output element at a time, straight from the definitions of the
pre-norm transformer layer that the tensor-parallel shard must reproduce
(undercodenews post 110319 on tensor parallelism, section "the Original":
Q/K/V projections split into heads, independent per-head attention, heads
concatenated, output projection; FFN of two linears with an activation).
The readings for what the pages leave open are the same as ``oracle.layer``
states (pre-norm, RMSNorm, rotate-half RoPE, GQA by contiguous groups,
SwiGLU or erf-GELU, residual once, bf16 storage points).
"""

from __future__ import annotations

import math


def _bf16(a: float) -> float:
    # Python's round() is round-half-to-even.
    if a == 0.0:
        return 0.0
    _, e = math.frexp(a)
    e = max(e, -125)
    q = math.ldexp(1.0, e - 8)
    return round(a / q) * q


def _rmsnorm_row(row, gamma, eps):
    acc = 0.0
    for v in row:
        acc += v * v
    scale = 1.0 / math.sqrt(acc / len(row) + eps)
    return [row[i] * scale * gamma[i] for i in range(len(row))]


def _matvec(Wm, vec):
    """out[o] = sum_i Wm[o][i] * vec[i]   (Wm stored [out][in])."""
    out = []
    for wrow in Wm:
        acc = 0.0
        for i in range(len(vec)):
            acc += wrow[i] * vec[i]
        out.append(acc)
    return out


def layer(x, W, *, hidden, heads, kv_heads, ffn, swiglu=True, norm=True,
          rope=True, eps=1e-5, theta=10000.0, mirror=False):
    """x: nested list [B][S][hidden]; W: dict of nested lists ([out][in]).
    Returns dict with 'h' and 'y' as nested lists [B][S][hidden]."""
    st = _bf16 if mirror else (lambda a: a)
    d = hidden // heads
    group = heads // kv_heads
    B, S = len(x), len(x[0])
    h_out, y_out = [], []
    for b in range(B):
        # per token: normalized input, projections (after rotation)
        qs, ks, vs = [], [], []
        for s in range(S):
            row = list(x[b][s])
            n = [st(v) for v in _rmsnorm_row(row, W["g1"], eps)] if norm else row
            q = _matvec(W["wq"], n)
            k = _matvec(W["wk"], n)
            v = _matvec(W["wv"], n)
            if rope:
                for (vec, nh) in ((q, heads), (k, kv_heads)):
                    for hh in range(nh):
                        base = hh * d
                        for i in range(d // 2):
                            ang = s * theta ** (-2.0 * i / d)
                            a, c = vec[base + i], vec[base + i + d // 2]
                            vec[base + i] = a * math.cos(ang) - c * math.sin(ang)
                            vec[base + i + d // 2] = c * math.cos(ang) + a * math.sin(ang)
            qs.append([st(a) for a in q])
            ks.append([st(a) for a in k])
            vs.append([st(a) for a in v])
        hb, yb = [], []
        for s in range(S):
            # attention of token s over tokens 0..s, head by head
            o = [0.0] * (heads * d)
            for hh in range(heads):
                g = hh // group
                scores = []
                for l in range(s + 1):
                    acc = 0.0
                    for i in range(d):
                        acc += qs[s][hh * d + i] * ks[l][g * d + i]
                    scores.append(acc / math.sqrt(d))
                m = max(scores)
                e = [math.exp(a - m) for a in scores]
                z = sum(e)
                for i in range(d):
                    acc = 0.0
                    for l in range(s + 1):
                        acc += e[l] / z * vs[l][g * d + i]
                    o[hh * d + i] = st(acc)
            a_out = _matvec(W["wo"], o)
            hrow = [st(x[b][s][i] + a_out[i]) for i in range(hidden)]
            n2 = [st(v) for v in _rmsnorm_row(hrow, W["g2"], eps)] if norm else hrow
            if swiglu:
                gt = _matvec(W["w_gate"], n2)
                up = _matvec(W["w_up"], n2)
                act = [st(gt[j] / (1.0 + math.exp(-gt[j])) * up[j]) for j in range(ffn)]
            else:
                z1 = _matvec(W["w_up"], n2)
                act = [st(0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0)))) for a in z1]
            m_out = _matvec(W["w_down"], act)
            hb.append(hrow)
            yb.append([st(hrow[i] + m_out[i]) for i in range(hidden)])
        h_out.append(hb)
        y_out.append(yb)
    return {"h": h_out, "y": y_out}
