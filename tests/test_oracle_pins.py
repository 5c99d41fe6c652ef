"""Pins of the CPU oracle to facts other than itself.

Every test here runs on the CPU.  Each one is chosen so that a plausible slip
in the oracle (a dropped scale, a mask on the wrong side of the diagonal, a
rotation applied to v or not to k, the wrong rotate-half pairing or sign, a
transposed operand in the backward, a bias with the wrong sign, documents that
leak) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import neox_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- rotation

def test_inv_freq_closed_form():
    # base^(-2p/rd) for the 20B rotary width 24: 10^(-p/3) when base = 1e4.
    f = orc.rope_inv_freq(24, 10000.0)
    assert f.shape == (12,)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[[3, 6, 9]], [0.1, 0.01, 0.001], rtol=1e-14)
    f128 = orc.rope_inv_freq(128, 10000.0)
    np.testing.assert_allclose(f128[32], 0.01, rtol=1e-14)  # 1e4^(-64/128)
    with pytest.raises(ValueError):
        orc.rope_inv_freq(5, 10000.0)


@pytest.mark.parametrize("rd,D", [(2, 8), (16, 64), (24, 96), (128, 128)])
def test_rotation_is_complex_multiplication(rd, D):
    """Rotate-half with pairs (p, p + rd/2): z_p = x_p + i x_{p+rd/2} times
    exp(i t w_p), w_p = base^(-2p/rd) computed here as exp(-2p/rd ln base)."""
    rng = np.random.default_rng(1)
    S = 37
    x = _rand(rng, 3, S, D)
    pos = np.arange(S)
    y = orc.rope_rotate(x, pos, rd, 10000.0)
    h = rd // 2
    w = np.exp(-(2.0 * np.arange(h) / rd) * math.log(10000.0))
    z = (x[..., :h] + 1j * x[..., h:rd]) * np.exp(1j * pos[:, None] * w[None, :])
    np.testing.assert_allclose(y[..., :h], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[..., h:rd], z.imag, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(y[..., rd:], x[..., rd:])  # pass-through dims


def test_rotation_identity_at_zero_and_rd0():
    rng = np.random.default_rng(2)
    x = _rand(rng, 1, 64)
    np.testing.assert_array_equal(orc.rope_rotate(x, [0], 64, 10000.0), x)
    x = _rand(rng, 10, 64)
    np.testing.assert_array_equal(orc.rope_rotate(x, np.arange(10), 0, 10000.0), x)


def test_rotation_preserves_norm_and_inverse():
    rng = np.random.default_rng(3)
    x = _rand(rng, 2, 50, 96)
    pos = np.arange(50) * 97 + 13
    y = orc.rope_rotate(x, pos, 24, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)
    back = orc.rope_rotate(y, pos, 24, 10000.0, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_rotation_relative_position():
    """(R_{m+t} q).(R_{n+t} k) = (R_m q).(R_n k): scores depend on m - n only."""
    rng = np.random.default_rng(4)
    q = _rand(rng, 1, 128)
    k = _rand(rng, 1, 128)
    for m, n, t in [(5, 2, 100), (0, 0, 1000), (300, 17, 4000), (9, 40, 16000)]:
        a = orc.rope_rotate(q, [m + t], 128, 1e4) @ orc.rope_rotate(k, [n + t], 128, 1e4).T
        b = orc.rope_rotate(q, [m], 128, 1e4) @ orc.rope_rotate(k, [n], 128, 1e4).T
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- forward closed forms

def test_hand_computed_two_tokens():
    """S=2, D=rd=2, scale 1: positions 0 and 1 rotate by 0 and 1 radian.

    q = [[a, 0], [0, 1]], k = [[1, 0], [0, 1]], v = [[1, 2], [3, 4]].
    Row 0 sees key 0 only: o0 = v0, lse0 = a.
    Row 1: q~1 = R_1 (0, 1) = (-sin 1, cos 1); k~0 = (1, 0);
    k~1 = R_1 (0, 1) = (-sin 1, cos 1), so s10 = -sin 1 and s11 = 1.
    """
    a = 0.3
    q = np.array([[[[a, 0.0], [0.0, 1.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    o, lse = orc.attn_fwd(q, k, v, rotary_dim=2, rope_base=10000.0, softmax_scale=1.0)
    s10, s11 = -math.sin(1.0), 1.0
    z = math.exp(s10) + math.exp(s11)
    p0, p1 = math.exp(s10) / z, math.exp(s11) / z
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 2.0], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [a, math.log(z)], atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], [p0 * 1 + p1 * 3, p0 * 2 + p1 * 4], atol=1e-15)


def test_single_token_returns_v():
    rng = np.random.default_rng(5)
    q, k, v = (_rand(rng, 2, 3, 1, 64) for _ in range(3))
    o, lse = orc.attn_fwd(q, k, v, rotary_dim=64, rope_base=1e4)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, np.sum(q * k, axis=-1) / 8.0, atol=1e-13)


@pytest.mark.parametrize("rd", [0, 16, 64])
def test_zero_query_gives_prefix_mean(rd):
    rng = np.random.default_rng(6)
    S, D = 40, 64
    q = np.zeros((1, 2, S, D))
    k, v = _rand(rng, 1, 2, S, D), _rand(rng, 1, 2, S, D)
    o, lse = orc.attn_fwd(q, k, v, rotary_dim=rd, rope_base=1e4)
    mean = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(o, mean, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), lse.shape),
                               atol=1e-13)


def test_zero_query_with_documents():
    rng = np.random.default_rng(7)
    S, D = 30, 16
    offs = np.array([[0, 7, 7, 19, 30], [0, 30, 30, 30, 30]], dtype=np.int32)
    q = np.zeros((2, 1, S, D))
    k, v = _rand(rng, 2, 1, S, D), _rand(rng, 2, 1, S, D)
    o, lse = orc.attn_fwd(q, k, v, rotary_dim=16, rope_base=1e4, doc_offsets=offs)
    for b in range(2):
        for i in range(S):
            start = max(x for x in offs[b] if x <= i)
            np.testing.assert_allclose(o[b, 0, i], v[b, 0, start:i + 1].mean(axis=0), atol=1e-13)
            np.testing.assert_allclose(lse[b, 0, i], math.log(i - start + 1), atol=1e-13)


def test_alibi_zero_query_geometric_mean():
    """q = 0 with ALiBi: weights exp(-m (i - j)), so lse_i is the log of a
    geometric series, ln((1 - r^(i+1)) / (1 - r)) with r = exp(-m)."""
    rng = np.random.default_rng(8)
    S, D, H = 25, 8, 4
    q = np.zeros((1, H, S, D))
    k, v = _rand(rng, 1, H, S, D), _rand(rng, 1, H, S, D)
    o, lse = orc.attn_fwd(q, k, v, rotary_dim=0, alibi=True)
    slopes = [2.0 ** (-2.0 * (h + 1)) for h in range(H)]  # 2^(-8(h+1)/4)
    for h, m in enumerate(slopes):
        r = math.exp(-m)
        for i in range(S):
            w = np.array([r ** (i - j) for j in range(i + 1)])
            np.testing.assert_allclose(o[0, h, i], w @ v[0, h, :i + 1] / w.sum(), atol=1e-13)
            np.testing.assert_allclose(lse[0, h, i], math.log((1 - r ** (i + 1)) / (1 - r)),
                                       atol=1e-13)


def test_alibi_slopes_closed_form():
    np.testing.assert_allclose(orc.alibi_slopes(8), [2.0 ** -(h + 1) for h in range(8)],
                               rtol=1e-15)
    s32 = orc.alibi_slopes(32)
    np.testing.assert_allclose(s32[[3, 7, 31]], [0.5, 0.25, 2.0 ** -8], rtol=1e-15)


def test_probability_rows_via_identity_values():
    """With D = S and v = I the output is P itself: rows are non-negative, sum
    to 1 and vanish above the diagonal."""
    rng = np.random.default_rng(9)
    S = 24
    q, k = _rand(rng, 1, 1, S, S), _rand(rng, 1, 1, S, S)
    v = np.eye(S)[None, None]
    P, _ = orc.attn_fwd(q, k, v, rotary_dim=8, rope_base=1e4)
    P = P[0, 0]
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(P[np.triu_indices(S, 1)] == 0.0)
    assert np.all(P[np.tril_indices(S)] > 0.0)


def test_constant_values_give_constant_output_and_zero_qk_grads():
    rng = np.random.default_rng(10)
    S, D = 33, 32
    q, k, do = (_rand(rng, 1, 2, S, D) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal(D), (1, 2, S, D)).copy()
    o, lse, dq, dk, dv = orc.attn_bwd(q, k, v, do, rotary_dim=16, rope_base=1e4)
    np.testing.assert_allclose(o, v, atol=1e-13)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def test_first_row_of_each_document_returns_v():
    rng = np.random.default_rng(11)
    S, D = 50, 16
    offs = np.array([[0, 1, 12, 40, 50]], dtype=np.int32)
    q, k, v = (_rand(rng, 1, 2, S, D) for _ in range(3))
    o, _ = orc.attn_fwd(q, k, v, rotary_dim=16, rope_base=1e4, doc_offsets=offs)
    for s in offs[0][:-1]:
        np.testing.assert_allclose(o[0, :, s], v[0, :, s], atol=1e-14)


def test_packed_documents_equal_separate_runs():
    """Packed output = concatenation of each document run on its own.  RoPE
    positions keep counting across documents in a row, but scores depend only
    on position differences, so a separate run (positions from 0) agrees."""
    rng = np.random.default_rng(12)
    S, D = 64, 32
    offs = np.array([[0, 10, 33, 64]], dtype=np.int32)
    q, k, v, do = (_rand(rng, 1, 3, S, D) for _ in range(4))
    for alibi in (False, True):
        full = orc.attn_bwd(q, k, v, do, rotary_dim=32, rope_base=1e4, alibi=alibi,
                            doc_offsets=offs)
        for a, b in zip(offs[0][:-1], offs[0][1:]):
            part = orc.attn_bwd(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], do[:, :, a:b],
                                rotary_dim=32, rope_base=1e4, alibi=alibi)
            for f, p in zip(full, part):
                np.testing.assert_allclose(f[:, :, a:b], p, atol=1e-10)


def test_rope_positions_restart_per_document():
    """Positions inside documents, by hand: [0,3) [3,3) [3,7) [7,10)."""
    offs = np.array([0, 3, 3, 7, 10])
    np.testing.assert_array_equal(orc.rope_positions(10, offs, True),
                                  [0, 1, 2, 0, 1, 2, 3, 0, 1, 2])
    np.testing.assert_array_equal(orc.rope_positions(10, offs, False), np.arange(10))
    np.testing.assert_array_equal(orc.rope_positions(10, None, True), np.arange(10))


def test_document_positions_equal_separate_runs_and_global_positions():
    """With positions restarted at each document, every document is rotated as
    if it stood alone: the packed run equals separate runs (positions from 0),
    forward and backward.  R_a^T R_b = R_(b-a), so shifting both positions of a
    pair by the document start changes no score: the global-position run
    agrees too (to rounding)."""
    rng = np.random.default_rng(21)
    S, D = 70, 32
    offs = np.array([[0, 17, 17, 50, 70]], dtype=np.int32)
    q, k, v, do = (_rand(rng, 1, 2, S, D) for _ in range(4))
    for rd in (8, 32):
        per_doc = orc.attn_bwd(q, k, v, do, rotary_dim=rd, rope_base=50.0, doc_offsets=offs,
                               rope_doc_positions=True)
        glob = orc.attn_bwd(q, k, v, do, rotary_dim=rd, rope_base=50.0, doc_offsets=offs)
        for f, g in zip(per_doc, glob):
            np.testing.assert_allclose(f, g, atol=1e-10)
        for a, b in zip(offs[0][:-1], offs[0][1:]):
            if a == b:
                continue
            part = orc.attn_bwd(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], do[:, :, a:b],
                                rotary_dim=rd, rope_base=50.0)
            for f, p in zip(per_doc, part):
                np.testing.assert_allclose(f[:, :, a:b], p, atol=1e-10)
        o, _ = orc.attn_fwd(q, k, v, rotary_dim=rd, rope_base=50.0, doc_offsets=offs,
                            rope_doc_positions=True)
        np.testing.assert_allclose(o, per_doc[0], atol=1e-12)


# ---------------------------------------------------------------- library special case

def _torch_reference(q, k, v, do, rd, base, causal, scale, slopes, offs):
    """torch float64: rotation via complex multiplication, attention via
    scaled_dot_product_attention with an explicit boolean or additive mask,
    gradients via autograd, lse via torch.logsumexp of the masked scores."""
    B, H, S, D = q.shape
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    tdo = torch.tensor(do, dtype=torch.float64)

    def rot(x):
        if rd == 0:
            return x
        h = rd // 2
        w = torch.exp(-(2.0 * torch.arange(h, dtype=torch.float64) / rd) * math.log(base))
        ang = torch.arange(S, dtype=torch.float64)[:, None] * w[None, :]
        z = torch.complex(x[..., :h], x[..., h:rd]) * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([z.real, z.imag, x[..., rd:]], dim=-1)

    qr, kr = rot(tq), rot(tk)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    allow = torch.ones(B, 1, S, S, dtype=torch.bool)
    if causal:
        allow = allow & (j <= i)
    if offs is not None:
        doc = torch.stack([torch.bucketize(torch.arange(S), torch.tensor(r[1:-1], dtype=torch.int64),
                                           right=True) for r in offs])
        allow = allow & (doc[:, None, :, None] == doc[:, None, None, :])
    mask = torch.zeros(B, H, S, S, dtype=torch.float64).masked_fill(~allow, float("-inf"))
    if slopes is not None:
        mask = mask + (-torch.tensor(slopes, dtype=torch.float64)[None, :, None, None]
                       * (i - j).to(torch.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qr, kr, tv, attn_mask=mask, scale=scale)
    o.backward(tdo)
    lse = torch.logsumexp(scale * qr.detach() @ kr.detach().transpose(-1, -2) + mask, dim=-1)
    return (o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


CASES = [
    # (B, H, S, D, rd, causal, alibi, docs)
    (1, 2, 1, 8, 8, True, False, None),
    (2, 3, 45, 64, 16, True, False, None),
    (1, 2, 70, 96, 24, True, False, None),
    (1, 2, 100, 128, 128, True, False, None),
    (1, 2, 64, 32, 0, True, True, None),
    (2, 4, 90, 32, 0, True, True, [[0, 20, 21, 64, 90], [0, 90, 90, 90, 90]]),
    (1, 2, 50, 32, 32, True, False, [[0, 17, 50]]),
    (1, 2, 40, 16, 8, False, False, None),
    (1, 2, 40, 16, 8, False, True, [[0, 15, 40]]),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_sdpa_float64(case):
    B, H, S, D, rd, causal, alibi, docs = case
    rng = np.random.default_rng(100 + S + D)
    q, k, v, do = (_rand(rng, B, H, S, D) for _ in range(4))
    offs = None if docs is None else np.array(docs, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    slopes = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)] if alibi else None
    ref = _torch_reference(q, k, v, do, rd, 1e4, causal, scale, slopes, offs)
    got = orc.attn_bwd(q, k, v, do, rotary_dim=rd, rope_base=1e4, causal=causal,
                       alibi=alibi, doc_offsets=offs)
    for name, r, g in zip(["o", "lse", "dq", "dk", "dv"], ref, got):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-11, err_msg=name)
    o_f, lse_f = orc.attn_fwd(q, k, v, rotary_dim=rd, rope_base=1e4, causal=causal,
                              alibi=alibi, doc_offsets=offs)
    np.testing.assert_array_equal(o_f, got[0])
    np.testing.assert_array_equal(lse_f, got[1])


def test_head_subset_equals_full_run():
    rng = np.random.default_rng(13)
    q, k, v, do = (_rand(rng, 2, 3, 20, 16) for _ in range(4))
    full = orc.attn_bwd(q, k, v, do, rotary_dim=8, rope_base=1e4)
    sub = orc.attn_bwd(q, k, v, do, rotary_dim=8, rope_base=1e4, heads=[(1, 2), (0, 1)])
    for f, s in zip(full, sub):
        np.testing.assert_array_equal(s[0], f[1, 2])
        np.testing.assert_array_equal(s[1], f[0, 1])


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("rd,alibi,docs,causal", [
    (0, False, None, True), (2, False, None, True), (4, False, None, True),
    (4, True, None, True), (2, True, [[0, 3, 7]], True), (4, False, [[0, 2, 7]], False),
])
def test_gradients_by_central_differences(rd, alibi, docs, causal):
    """L = sum(o * dO); dL/dx by central differences (h = 1e-6) on every
    element of q, k, v at B = H = 1, S = 7, D = 4."""
    rng = np.random.default_rng(14 + rd)
    S, D = 7, 4
    q, k, v, do = (_rand(rng, 1, 1, S, D) for _ in range(4))
    offs = None if docs is None else np.array(docs, dtype=np.int32)
    kw = dict(rotary_dim=rd, rope_base=100.0, causal=causal, alibi=alibi, doc_offsets=offs)
    _, _, dq, dk, dv = orc.attn_bwd(q, k, v, do, **kw)

    def loss(qq, kk, vv):
        o, _ = orc.attn_fwd(qq, kk, vv, **kw)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


# ---------------------------------------------------------------- gradient invariants

def test_gradient_sums_per_document():
    """Rows of P sum to 1 inside a document, so sum_j dv_j = sum_i dO_i per
    document; rows of dS sum to 0, so sum_j R_j dk_j = 0 per document."""
    rng = np.random.default_rng(15)
    S, D = 80, 32
    offs = np.array([[0, 25, 26, 80]], dtype=np.int32)
    q, k, v, do = (_rand(rng, 1, 2, S, D) for _ in range(4))
    _, _, dq, dk, dv = orc.attn_bwd(q, k, v, do, rotary_dim=32, rope_base=1e4,
                                    alibi=True, doc_offsets=offs)
    kr_grad = orc.rope_rotate(dk, np.arange(S), 32, 1e4)  # R_j dk_j = dk~_j
    for a, b in zip(offs[0][:-1], offs[0][1:]):
        np.testing.assert_allclose(dv[:, :, a:b].sum(axis=2), do[:, :, a:b].sum(axis=2),
                                   atol=1e-11)
        np.testing.assert_allclose(kr_grad[:, :, a:b].sum(axis=2), 0.0, atol=1e-11)


def test_zero_output_gradient_gives_zero_gradients():
    rng = np.random.default_rng(16)
    q, k, v = (_rand(rng, 1, 2, 30, 16) for _ in range(3))
    _, _, dq, dk, dv = orc.attn_bwd(q, k, v, np.zeros_like(q), rotary_dim=16, rope_base=1e4)
    assert not dq.any() and not dk.any() and not dv.any()


# ---------------------------------------------------------------- page facts

def test_neox20b_head_layout_fixture():
    """The 20B layout printed on the FasterTransformer GPT-NeoX guide, section
    on the model configuration: 64 heads of 96 dims (hidden 6144), 24 rotary
    dims; the GPT-NeoX-20B release note gives the 2048-token context."""
    with open(os.path.join(GOLDEN, "neox20b_layout.json")) as f:
        fx = json.load(f)
    assert fx["head_num"] * fx["size_per_head"] == fx["hidden"] == 6144
    from causal_attention_neox_amd.workloads import WORKLOADS
    wl = WORKLOADS["neox20b_s2048_h64_d96_rd24"]
    assert (wl.H, wl.D, wl.rotary_dim, wl.S) == (
        fx["head_num"], fx["size_per_head"], fx["rotary_embedding"], fx["context_tokens"])
    # 24 rotary dims of 96: 12 rotary pairs, dims 24..95 pass through
    x = np.random.default_rng(17).standard_normal((5, 96))
    y = orc.rope_rotate(x, np.arange(5), fx["rotary_embedding"], 1e4)
    np.testing.assert_array_equal(y[:, 24:], x[:, 24:])
    assert not np.allclose(y[1:, :24], x[1:, :24])


def test_oracle_regression_fixture():
    """Values written by tests/golden/make_golden.py, which calls only the
    oracle on inputs it builds itself; guards later edits of the oracle."""
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        inp = {n: np.array(case[n], dtype=np.float64) for n in ("q", "k", "v", "dout")}
        offs = None if case["doc_offsets"] is None else np.array(case["doc_offsets"], np.int32)
        got = orc.attn_bwd(inp["q"], inp["k"], inp["v"], inp["dout"],
                           rotary_dim=case["rotary_dim"], rope_base=case["rope_base"],
                           causal=case["causal"], alibi=case["alibi"], doc_offsets=offs)
        for name, g in zip(["o", "lse", "dq", "dk", "dv"], got):
            np.testing.assert_allclose(g, np.array(case[name]), rtol=1e-12, atol=1e-12,
                                       err_msg=f"{case['name']}:{name}")


@pytest.mark.parametrize("rd,D,t", [(16, 64, 0), (24, 96, 5), (128, 128, 40), (0, 64, 17)])
def test_decode_step_is_the_last_causal_row(rd, D, t):
    """A decoding step over a cache of t rotated keys equals row t of causal
    attention over the t + 1 tokens (computed by the full-matrix path, which is
    itself pinned to torch's float64 SDPA)."""
    rng = np.random.default_rng(500 + t)
    q, k, v = (_rand(rng, t + 1, D) for _ in range(3))
    k_cache = orc.rope_rotate(k[:t], np.arange(t), rd, 10000.0)
    o, lse, k_rot = orc.attn_decode(q[t], k[t], v[t], k_cache, v[:t], rotary_dim=rd)
    of, lf = orc.attn_fwd(q[None, None], k[None, None], v[None, None], rotary_dim=rd)
    np.testing.assert_allclose(o, of[0, 0, t], rtol=0, atol=1e-12)
    assert abs(lse - lf[0, 0, t]) < 1e-12


def test_decode_first_token_returns_v():
    """Position 0 leaves q and k unrotated; with one token the output is v and
    the logsumexp is the single score scale * q . k."""
    rng = np.random.default_rng(510)
    q, k, v = (_rand(rng, 96) for _ in range(3))
    o, lse, k_rot = orc.attn_decode(q, k, v, np.zeros((0, 96)), np.zeros((0, 96)),
                                    rotary_dim=24)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    assert abs(lse - float(q @ k) / math.sqrt(96)) < 1e-12
    np.testing.assert_allclose(k_rot, k, rtol=0, atol=1e-15)


def test_decode_appended_key_is_rotated_at_its_position():
    """The appended key is k times exp(i t w_p) in the complex pair form."""
    rng = np.random.default_rng(511)
    rd, D, t = 24, 96, 33
    q, k, v = (_rand(rng, D) for _ in range(3))
    k_cache, v_cache = _rand(rng, t, D), _rand(rng, t, D)
    _, _, k_rot = orc.attn_decode(q, k, v, k_cache, v_cache, rotary_dim=rd)
    h = rd // 2
    w = np.exp(-(2.0 * np.arange(h) / rd) * math.log(10000.0))
    z = (k[:h] + 1j * k[h:rd]) * np.exp(1j * t * w)
    np.testing.assert_allclose(k_rot[:h], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(k_rot[h:rd], z.imag, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(k_rot[rd:], k[rd:])


# ---------------------------------------------------------------- FP8 (E4M3)

def test_e4m3_decode_format_constants():
    """Values fixed by the E4M3 definition: 1.0, the largest finite value
    448 = 1.75 x 2^8, the smallest normal 2^-6, the smallest subnormal 2^-9,
    signed zero, NaN codes, and 0.5 / 3.0 / -2.25."""
    d = orc.e4m3_decode
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x00) == 0.0 and d(0x80) == 0.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x30) == 0.5 and d(0x44) == 3.0 and d(0xC1) == -2.25


def test_e4m3_decode_is_monotonic_with_three_mantissa_bits():
    """Positive finite codes 0..126 decode to strictly increasing values; inside
    each binade there are 8 evenly spaced values (3 mantissa bits)."""
    v = orc.e4m3_decode(np.arange(127))
    assert np.all(np.diff(v) > 0)
    for e in range(1, 16):
        block = v[8 * e: 8 * e + 8] if 8 * e + 8 <= 127 else v[8 * e: 127]
        steps = np.diff(block)
        np.testing.assert_allclose(steps, 2.0 ** (e - 7) / 8)


def test_fp8_forward_is_attention_of_dequantised_inputs():
    """The FP8 forward equals the exact forward over code x scale, with the
    scales entering linearly: doubling v's scale doubles o, and halving q's
    scale while doubling k's leaves everything unchanged."""
    rng = np.random.default_rng(31)
    B, H, S, D = 1, 2, 40, 16
    q8, k8, v8 = (rng.integers(0, 256, (B, H, S, D)) for _ in range(3))
    for c in (q8, k8, v8):
        c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
        c[(c & 0x78) > 0x58] &= 0xBF   # keep magnitudes moderate (exponent <= 11)
    o, lse = orc.attn_fwd_fp8(q8, k8, v8, 0.05, 0.1, 0.5)
    qd, kd, vd = (orc.e4m3_decode(c) * s for c, s in ((q8, 0.05), (k8, 0.1), (v8, 0.5)))
    o2, lse2 = orc.attn_fwd(qd, kd, vd, rotary_dim=0)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    o3, lse3 = orc.attn_fwd_fp8(q8, k8, v8, 0.05, 0.1, 1.0)
    np.testing.assert_allclose(o3, 2.0 * o, atol=1e-12)
    o4, lse4 = orc.attn_fwd_fp8(q8, k8, v8, 0.025, 0.2, 0.5)
    np.testing.assert_allclose(o4, o, atol=1e-12)
    np.testing.assert_allclose(lse4, lse, atol=1e-12)
