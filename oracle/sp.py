"""Sequence-parallel variant of the shard: TEST INFRASTRUCTURE ONLY.

undercodenews post 110319 on tensor parallelism in transformers, section
"What Undercode Say": production systems pair tensor parallelism with
sequence parallelism.  The pages give no algorithm for it, so the reading
taken here is the standard one for a sequential pre-norm block:

1. between the two stages the activations are split by token: rank r holds
   rows [r T/t, (r+1) T/t) of the flattened [T = B*S, hidden] tensor, and
   T must divide by t;
2. the all-reduce of a stage's partials becomes a reduce-scatter: rank r
   receives its rows of the rank-order sum, plus its rows of the residual,
   stored at the activation precision;
3. each rank normalises only its rows (RMSNorm is a per-token operation),
   and an all-gather of the normalised rows rebuilds the full stage input of
   the next column-parallel projection, whose stage then skips its norm.

Because every step is row-wise or a permutation of the plain layer's, the
ranks' outputs concatenate to the plain layer's result exactly.
"""

from __future__ import annotations

import numpy as np

from .layer import Spec, _store, attn_from_n1, check_partition, mlp_from_n2, norm1, norm2


def token_rows(T: int, t: int, r: int) -> slice:
    """Rows of the flattened token dimension owned by rank r."""
    if T % t:
        raise ValueError("the token count must divide by the tp degree")
    n = T // t
    return slice(r * n, (r + 1) * n)


def reduce_scatter(partials, residual_rows, spec: Spec, t: int, r: int):
    """Rank r's rows of (sum of the rank partials in rank order) + its rows
    of the residual.  partials: t arrays [T, hidden] (any leading shape that
    flattens to T rows); residual_rows [T/t, hidden]."""
    flat = [np.asarray(p, np.float64).reshape(-1, spec.hidden) for p in partials]
    rows = token_rows(flat[0].shape[0], t, r)
    s = np.zeros_like(flat[0][rows])
    for p in flat:
        s = s + p[rows]
    return _store(spec, s + np.asarray(residual_rows, np.float64).reshape(s.shape))


def all_gather(pieces) -> np.ndarray:
    """Rank-order concatenation of the ranks' row blocks."""
    return np.concatenate([np.asarray(p, np.float64) for p in pieces], axis=0)


def layer_sp(x, W, spec: Spec, t: int):
    """The sequence-parallel layer as t ranks compute it.  x [B, S, hidden];
    returns per-rank row blocks (x_r, n1_r, h_r, n2_r, y_r, each [T/t, hidden]),
    the gathered stage inputs and every rank's stage outputs."""
    check_partition(spec, t)
    x = np.asarray(x, np.float64)
    B, S, h = x.shape
    T = B * S
    xf = x.reshape(T, h)
    xs = [xf[token_rows(T, t, r)] for r in range(t)]
    n1s = [norm1(xr, W, spec) for xr in xs]
    n1 = all_gather(n1s).reshape(B, S, h)
    attn = [attn_from_n1(n1, W, spec, t, r) for r in range(t)]
    hs = [reduce_scatter([a["partial"] for a in attn], xs[r], spec, t, r) for r in range(t)]
    n2s = [norm2(hr, W, spec) for hr in hs]
    n2 = all_gather(n2s).reshape(B, S, h)
    mlp = [mlp_from_n2(n2, W, spec, t, r) for r in range(t)]
    ys = [reduce_scatter([m["partial"] for m in mlp], hs[r], spec, t, r) for r in range(t)]
    return {"x": xs, "n1": n1s, "n1_full": n1, "attn": attn, "h": hs, "n2": n2s, "n2_full": n2,
            "mlp": mlp, "y": ys}
