"""Pins of the sequence-parallel oracle (oracle/sp.py): the row split and
rejoin are exact permutations of the plain layer's arithmetic, so the ranks'
outputs must concatenate to it exactly; a planted mistake in the row
bookkeeping must break that."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import layer as O
from oracle import sp
from tensor_transformer_layer_tp_amd import synth


def _case(mirror, swiglu=True, norm=True, B=2, S=6, kv=2):
    spec = O.Spec(64, 4, kv, 128, swiglu=swiglu, norm=norm, mirror_bf16=mirror)
    raw = synth.draw_layer(64, 4, kv, 128, swiglu=swiglu, batch=B, seq=S, seed=17)
    raw["g1"] = 1 + synth.draw_normal((64,), 18, 0.1)
    raw["g2"] = 1 + synth.draw_normal((64,), 19, 0.1)
    x = raw.pop("x")
    return spec, raw, x


@pytest.mark.parametrize("mirror", [False, True])
@pytest.mark.parametrize("t,kv", [(1, 2), (2, 2), (4, 4)])
def test_sp_layer_equals_plain_layer(mirror, t, kv):
    spec, W, x = _case(mirror, kv=kv)
    ref = O.layer(x, W, spec, t)
    out = sp.layer_sp(x, W, spec, t)
    T = x.shape[0] * x.shape[1]
    assert np.array_equal(np.concatenate(out["h"]), ref["h"].reshape(T, -1))
    assert np.array_equal(np.concatenate(out["y"]), ref["y"].reshape(T, -1))
    # the gathered stage inputs are the plain stages' normalised inputs
    assert np.array_equal(out["n1_full"], ref["attn"][0]["n1"])
    assert np.array_equal(out["n2_full"], ref["mlp"][0]["n2"])


def test_sp_gelu_without_norm():
    spec, W, x = _case(False, swiglu=False, norm=False, B=1, S=8)
    ref = O.layer(x, W, spec, 2)
    out = sp.layer_sp(x, W, spec, 2)
    assert np.array_equal(np.concatenate(out["y"]), ref["y"].reshape(8, -1))


def test_reduce_scatter_rows_and_gather_inverse():
    spec = O.Spec(64, 4, 2, 128, mirror_bf16=False)
    parts = [synth.draw_normal((12, 64), 30 + i) for i in range(3)]
    res = synth.draw_normal((12, 64), 40)
    full = O.reduce(parts, res, spec)
    pieces = [sp.reduce_scatter(parts, res[sp.token_rows(12, 3, r)], spec, 3, r) for r in range(3)]
    assert np.array_equal(sp.all_gather(pieces), full)
    with pytest.raises(ValueError):
        sp.token_rows(10, 3, 0)


def test_planted_row_offset_is_caught():
    """Taking rank r's residual rows from the wrong block changes the result."""
    spec, W, x = _case(False)
    ref = O.layer(x, W, spec, 2)
    out = sp.layer_sp(x, W, spec, 2)
    parts = [a["partial"] for a in out["attn"]]
    xs = out["x"]
    wrong = [sp.reduce_scatter(parts, xs[1 - r], spec, 2, r) for r in range(2)]
    assert not np.allclose(np.concatenate(wrong), ref["h"].reshape(12, -1))
