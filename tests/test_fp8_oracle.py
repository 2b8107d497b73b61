"""Pins of the E4M3 oracle (oracle/fp8.py) against what the format and the
mathematics fix: torch's float8_e4m3fn conversions (a library implementation
of the same OCP format), hand cases from the format definition, the
quantisation's invariants and its error bound."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import layer as O
from tensor_transformer_layer_tp_amd import synth


def torch_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ov, tv = fp8.e4m3_value(codes), torch_value(codes)
    assert np.array_equal(np.isnan(ov), np.isnan(tv))
    assert np.isnan(ov).sum() == 2                      # S.1111.111 only: no infinities
    ok = ~np.isnan(tv)
    assert np.array_equal(ov[ok], tv[ok])


@pytest.mark.parametrize("v,code", [
    (448.0, 0x7E), (-448.0, 0xFE),       # largest finite: 1.75 * 2^8
    (1.0, 0x38), (-1.0, 0xB8), (240.0, 0x77),
    (2.0 ** -6, 0x08),                   # smallest normal
    (2.0 ** -9, 0x01),                   # smallest subnormal
    (7 * 2.0 ** -9, 0x07),               # largest subnormal
    (0.5 * 2.0 ** -9, 0x00),             # tie between 0 and 2^-9 -> even code 0
    (1.5 * 2.0 ** -9, 0x02),             # tie between codes 1 and 2 -> 2
    (1.0625, 0x38),                      # tie between 1 and 1.125 -> 1 (even mantissa)
    (1.1875, 0x3A),                      # tie between 1.125 and 1.25 -> 1.25
    (0.0, 0x00), (-0.0, 0x80),
])
def test_encode_hand_cases(v, code):
    assert int(fp8.e4m3_encode(np.array([v], np.float32))[0]) == code


def test_encode_matches_library_on_values_ties_and_random():
    vals = fp8._POS_VALUES
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(3)
    v = np.concatenate([vals, -vals, mids, -mids, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 0.05,
                        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000)]).astype(np.float32)
    v = np.clip(v, -448, 448)
    assert np.array_equal(fp8.e4m3_encode(v), torch_encode(v))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))


def test_quantize_rows_invariants_and_error_bound():
    w = synth.draw_normal((64, 1024), 5, 0.02)
    w[3] = 0.0
    w[5, :] *= 1e-30                                     # tiny row: scale in fp32's low range
    codes, scale = fp8.quantize_rows(w)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[3] == 1.0 and not codes[3].any()
    vals = fp8.e4m3_value(codes)
    nz = np.array([r != 3 for r in range(64)])
    assert np.all(np.max(np.abs(vals[nz]), axis=1) == 448.0)   # every nonzero row reaches the largest code
    q = np.asarray(w, np.float32) / scale[:, None]
    err = np.abs(q.astype(np.float64) - vals)
    bound = np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10)    # half an E4M3 spacing
    assert np.all(err <= bound * (1 + 1e-6))
    wq = fp8.dequantize_rows(codes, scale)
    assert np.all(np.sign(wq) * np.sign(w) >= 0)


def test_rank_weights_touch_only_the_rank_blocks():
    spec = O.Spec(256, 4, 2, 512)
    W = {k: v for k, v in synth.draw_layer(256, 4, 2, 512, seed=7).items()}
    t, r = 2, 1
    Wq = fp8.rank_weights(W, spec, t, r)
    hb, kb, fb = O.rank_blocks(spec, t, r)
    d = spec.head_dim
    own_q, own_k = slice(hb.start * d, hb.stop * d), slice(kb.start * d, kb.stop * d)
    other_q = slice(0, hb.start * d)
    assert np.array_equal(Wq["wq"][other_q], W["wq"][other_q])
    assert not np.array_equal(Wq["wq"][own_q], W["wq"][own_q])
    assert np.array_equal(Wq["wo"][:, other_q], W["wo"][:, other_q])
    assert np.array_equal(Wq["w_down"][:, :fb.start], W["w_down"][:, :fb.start])
    assert np.array_equal(Wq["g1"], W["g1"])
    # column-parallel rows keep their own per-row scale whether sliced or not
    full = fp8.rank_weights(W, spec, 1, 0)
    assert np.array_equal(full["wk"][own_k], Wq["wk"][own_k])
    # quantised weights stay within the E4M3 relative error of the originals
    rel = np.abs(Wq["w_up"][fb.start:fb.stop] - W["w_up"][fb.start:fb.stop]).max() / np.abs(W["w_up"]).max()
    assert 0 < rel < 2.0 ** -4
