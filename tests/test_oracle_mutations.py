"""Planted mistakes in the oracle must trip at least one pin.

Each case monkeypatches one helper of ``oracle.neox_oracle`` (on the CPU, for
the duration of the test only) with a plausible slip, then runs the pin tests
of ``test_oracle_pins`` and expects at least one of them to fail.
"""

import numpy as np
import pytest

from oracle import neox_oracle as orc
from tests import test_oracle_pins as pins

ORIG = {n: getattr(orc, n) for n in
        ("rope_rotate", "rope_inv_freq", "allowed_mask", "alibi_bias", "_head_probs",
         "head_backward", "head_forward", "alibi_slopes", "attn_decode", "rope_positions",
         "e4m3_decode")}


def _rotate_sign_flipped(x, positions, rotary_dim, base, inverse=False):
    return ORIG["rope_rotate"](x, positions, rotary_dim, base, inverse=not inverse)


def _rotate_interleaved(x, positions, rotary_dim, base, inverse=False):
    x = np.asarray(x, dtype=np.float64)
    rd = int(rotary_dim)
    if rd == 0:
        return x.copy()
    th = orc.rope_angles(positions, rd, base) * (-1.0 if inverse else 1.0)
    c, s = np.cos(th), np.sin(th)
    y = x.copy()
    y[..., 0:rd:2] = x[..., 0:rd:2] * c - x[..., 1:rd:2] * s
    y[..., 1:rd:2] = x[..., 1:rd:2] * c + x[..., 0:rd:2] * s
    return y


def _inv_freq_missing_two(rotary_dim, base):
    p = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(base), -p / rotary_dim)


def _mask_strict(S, causal, offsets_row):
    m = ORIG["allowed_mask"](S, causal, offsets_row)
    np.fill_diagonal(m, S == 1)
    return m


def _mask_anticausal(S, causal, offsets_row):
    return ORIG["allowed_mask"](S, causal, offsets_row).T.copy()


def _mask_ignores_docs(S, causal, offsets_row):
    return ORIG["allowed_mask"](S, causal, None)


def _bias_wrong_sign(S, slope):
    return -ORIG["alibi_bias"](S, slope)


def _slopes_off_by_one(H):
    h = np.arange(H, dtype=np.float64)
    return np.power(2.0, -8.0 * h / H)


def _probs_scale_dropped(qr, kr, scale, bias, allowed):
    return ORIG["_head_probs"](qr, kr, 1.0, bias, allowed)


def _make_backward(variant):
    def head_backward(q, k, v, dout, *, rotary_dim, rope_base, causal, scale, slope=None,
                      offsets_row=None, positions=None):
        S = q.shape[0]
        pos = np.arange(S) if positions is None else positions
        qr = orc.rope_rotate(q, pos, rotary_dim, rope_base)
        kr = orc.rope_rotate(k, pos, rotary_dim, rope_base)
        bias = orc.alibi_bias(S, slope) if slope is not None else None
        P, lse = orc._head_probs(qr, kr, scale, bias, orc.allowed_mask(S, causal, offsets_row))
        o = P @ v
        dv = (P @ dout) if variant == "dv_untransposed" else (P.T @ dout)
        dP = dout @ v.T
        delta = np.sum(dout * (v if variant == "delta_uses_v" else o), axis=1)
        dS = P * (dP - delta[:, None])
        dqr = scale * (dS @ kr)
        dkr = scale * ((dS @ qr) if variant == "dk_untransposed" else (dS.T @ qr))
        inv = variant != "no_inverse_rotation"
        dq = orc.rope_rotate(dqr, pos, rotary_dim, rope_base, inverse=inv)
        dk = orc.rope_rotate(dkr, pos, rotary_dim, rope_base, inverse=inv)
        return o, lse, dq, dk, dv
    return head_backward


def _forward_rotates_v(q, k, v, *, rotary_dim, rope_base, causal, scale, slope=None,
                       offsets_row=None, positions=None):
    pos = np.arange(q.shape[0]) if positions is None else positions
    vr = ORIG["rope_rotate"](v, pos, rotary_dim, rope_base)
    return ORIG["head_forward"](q, k, vr, rotary_dim=rotary_dim, rope_base=rope_base,
                                causal=causal, scale=scale, slope=slope,
                                offsets_row=offsets_row, positions=positions)


def _forward_k_unrotated(q, k, v, *, rotary_dim, rope_base, causal, scale, slope=None,
                         offsets_row=None, positions=None):
    S = q.shape[0]
    pos = np.arange(S) if positions is None else positions
    qr = orc.rope_rotate(q, pos, rotary_dim, rope_base)
    bias = orc.alibi_bias(S, slope) if slope is not None else None
    P, lse = orc._head_probs(qr, k, scale, bias, orc.allowed_mask(S, causal, offsets_row))
    return P @ v, lse


def _decode_position_off_by_one(q, k, v, k_cache, v_cache, *, rotary_dim, rope_base=10000.0,
                                softmax_scale=None):
    t = int(np.asarray(k_cache).shape[0])
    D = np.asarray(q).shape[-1]
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    pos = np.array([max(t - 1, 0)])  # slip: the previous token's position
    qr = orc.rope_rotate(np.asarray(q, dtype=np.float64)[None], pos, rotary_dim, rope_base)[0]
    kr = orc.rope_rotate(np.asarray(k, dtype=np.float64)[None], pos, rotary_dim, rope_base)[0]
    keys = np.concatenate([np.asarray(k_cache, dtype=np.float64).reshape(t, D), kr[None]])
    vals = np.concatenate([np.asarray(v_cache, dtype=np.float64).reshape(t, D),
                           np.asarray(v, dtype=np.float64)[None]])
    s = scale * (keys @ qr)
    m = s.max()
    e = np.exp(s - m)
    return (e / e.sum()) @ vals, m + np.log(e.sum()), kr


def _positions_off_by_one_at_documents(S, offsets_row=None, per_document=False):
    pos = ORIG["rope_positions"](S, offsets_row, per_document)
    return np.where(pos > 0, pos - 1, pos) if per_document else pos  # slip: start at -1 / 0 twice


def _e4m3_bias_eight(codes):
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return ORIG["e4m3_decode"](c) / 2.0 * np.where((c >> 3) & 0xF, 1.0, 2.0)  # slip: bias 8


def _e4m3_no_subnormals(codes):
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where((c >> 3) & 0xF, ORIG["e4m3_decode"](c), 0.0)  # slip: subnormals flushed


MUTATIONS = {
    "rotation_sign": ("rope_rotate", _rotate_sign_flipped),
    "rotation_interleaved": ("rope_rotate", _rotate_interleaved),
    "inv_freq_exponent": ("rope_inv_freq", _inv_freq_missing_two),
    "mask_excludes_diagonal": ("allowed_mask", _mask_strict),
    "mask_anticausal": ("allowed_mask", _mask_anticausal),
    "mask_ignores_documents": ("allowed_mask", _mask_ignores_docs),
    "alibi_bias_sign": ("alibi_bias", _bias_wrong_sign),
    "alibi_slope_index": ("alibi_slopes", _slopes_off_by_one),
    "scale_dropped": ("_head_probs", _probs_scale_dropped),
    "dv_untransposed": ("head_backward", _make_backward("dv_untransposed")),
    "dk_untransposed": ("head_backward", _make_backward("dk_untransposed")),
    "delta_uses_v": ("head_backward", _make_backward("delta_uses_v")),
    "no_inverse_rotation": ("head_backward", _make_backward("no_inverse_rotation")),
    "v_rotated": ("head_forward", _forward_rotates_v),
    "k_unrotated": ("head_forward", _forward_k_unrotated),
    "decode_position_off_by_one": ("attn_decode", _decode_position_off_by_one),
    "document_positions_slip": ("rope_positions", _positions_off_by_one_at_documents),
    "e4m3_exponent_bias": ("e4m3_decode", _e4m3_bias_eight),
    "e4m3_flushes_subnormals": ("e4m3_decode", _e4m3_no_subnormals),
}


def _pin_calls():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        if name == "test_oracle_regression_fixture":
            continue  # stored oracle values would catch anything; use the real pins
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        argnames = [a.strip() for a in params[0].args[0].split(",")]
        for values in params[0].args[1]:
            values = values if len(argnames) > 1 else (values,)
            calls.append((name, fn, dict(zip(argnames, values))))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    attr, fake = MUTATIONS[mutation]
    monkeypatch.setattr(orc, attr, fake)
    caught = []
    for name, fn, kwargs in _pin_calls():
        try:
            with np.errstate(all="ignore"):
                fn(**kwargs)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(name)
    assert caught, f"no pin caught the planted mistake {mutation}"
