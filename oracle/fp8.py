"""FP8 (OCP E4M3) weight-only quantisation of a rank's decode weights.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages name quantisation only as the alternative to splitting a model
that does not fit (netray glossary "What Is Tensor Parallelism?", sections
"Tensor Parallelism Explained" and "In Practice": quantise first, shard only
if it still does not fit; byteledger "Tensor Parallelism: Splitting One
Layer Across GPUs", section "FAQ").  They fix no format or scheme, so the
readings taken here are:

1. format: OCP 8-bit floating point E4M3 -- 1 sign bit, 4 exponent bits
   (bias 7), 3 mantissa bits; exponent field 0 holds the subnormals
   m * 2^-9, fields 1..15 hold (1 + m/8) * 2^(e-7) except S.1111.111, which
   is NaN; there are no infinities; the largest finite value is 448;
2. scheme: one fp32 scale per output row of the rank's own weight slice
   (for the row-parallel W_o and W_down that is a row of the rank's column
   block), scale = fp32(max |w|) / fp32(448) (1 for an all-zero row); the
   code of w is the E4M3 value nearest to fp32(w) / scale computed in fp32,
   ties to the even code, the quotient first clamped to [-448, 448];
3. use: the decode projections read w' = value(code) * scale in place of w
   (activations, KV cache and every storage point stay as in bf16 decode).
"""

from __future__ import annotations

import numpy as np

from .layer import Spec, rank_blocks

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Real value of each E4M3 code (NaN for S.1111.111), as float64."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes and their values, ascending (code order is value order)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_encode(v) -> np.ndarray:
    """Code of the E4M3 value nearest to each element of v (|v| <= 448),
    ties to the even code, sign bit = sign of v (so -0.0 and negative values
    that round to zero give 0x80): a search in the table of representable
    values."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)   # the sign bit is v's sign


def quantize_rows(w):
    """Per-row E4M3 quantisation of w [N, K] (its values are taken as fp32).
    Returns (codes uint8 [N, K], scales float32 [N])."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (w32 / scale[:, None]).astype(np.float32)                 # fp32 quotient
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(q), scale


def dequantize_rows(codes, scales) -> np.ndarray:
    return e4m3_value(codes) * np.asarray(scales, np.float64)[:, None]


def _requant(w):
    c, s = quantize_rows(w)
    return dequantize_rows(c, s)


def rank_weights(W, spec: Spec, t: int, r: int) -> dict:
    """W with rank r's decode projection weights replaced by their
    dequantised E4M3 values (the other ranks' blocks and the norm gains are
    left as they are), so that the bf16 stage functions compute the fp8
    shard's decode."""
    hb, kb, fb = rank_blocks(spec, t, r)
    d = spec.head_dim
    out = {k: np.array(v, dtype=np.float64, copy=True) for k, v in W.items()}
    qrows = slice(hb.start * d, hb.stop * d)
    krows = slice(kb.start * d, kb.stop * d)
    cols = slice(fb.start, fb.stop)
    out["wq"][qrows] = _requant(out["wq"][qrows])
    out["wk"][krows] = _requant(out["wk"][krows])
    out["wv"][krows] = _requant(out["wv"][krows])
    out["wo"][:, qrows] = _requant(out["wo"][:, qrows])
    if spec.swiglu:
        out["w_gate"][cols] = _requant(out["w_gate"][cols])
    out["w_up"][cols] = _requant(out["w_up"][cols])
    out["w_down"][:, cols] = _requant(out["w_down"][:, cols])
    return out
