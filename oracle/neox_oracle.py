"""Plain double-precision CPU oracle for causal NeoX-rotary attention.

TEST INFRASTRUCTURE ONLY.  This module is imported only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The library (``causal_attention_neox_amd``) never imports, calls or links it, and
it imports nothing from the library: the two share no code.

What it computes, and where that comes from:

* The attention is exact: the GPT-NeoX pages say FlashAttention-2 is an exact
  attention algorithm that leaves the mathematical result unchanged and only
  changes tiling and IO ("GPT-NeoX 开源训练框架深度解读", section
  "问题二：注意力计算太慢").  So the oracle is the plain definition: the full
  score matrix of each head, a row-wise softmax, and the matrix products, with
  no tiling and no online rescaling.
* Rotary position embedding in the NeoX style is applied to both queries and
  keys ("FasterTransformer GPT-NeoX 推理指南", the GptNeoX.h facts
  ``neox_rotary_style_ true`` and section "模型配置": ``rotary_embedding 24``
  of ``size_per_head 96``, Q and K both rotated).  Only the first
  ``rotary_dim`` dims rotate; the frequencies are one per rotary pair, the
  ``attention.rotary_emb.inv_freq`` buffer of the same page's checkpoint list.
* ALiBi is the alternative position scheme ("GPT-NeoX 开源训练框架深度解读",
  section "架构创新").
* Autoregressive language modelling means causal attention (GPT-NeoX tool page,
  first paragraph; "GPT-NeoX: Как 20-миллиардная модель", section
  "Ключевые особенности и архитектура").

Readings taken where the pages are silent (each is also listed with the design
notes of this repository):
  R1  rotate-half pairing: dim p pairs with p + rotary_dim/2 (not GPT-J's
      interleaved 2p, 2p+1);
  R2  rotation sign: y_p = x_p cos - x_{p+h} sin, y_{p+h} = x_{p+h} cos + x_p sin,
      i.e. multiplication of (x_p + i x_{p+h}) by exp(+i theta);
  R3  theta[t, p] = t * base^(-2p / rotary_dim): the frequency denominator is
      rotary_dim, positions are 0..S-1 in each batch row;
  R4  scores s_ij = scale * (q~_i . k~_j) + bias_ij, the ALiBi bias added after
      scaling and not scaled; bias_ij = -slope_h * (i - j);
  R5  ALiBi slope of head h (0-based) is 2^(-8 (h+1) / H);
  R6  allowed(i, j) <=> (not causal or j <= i) and doc(i) == doc(j); the
      diagonal is allowed, so every row has at least one key;
  R7  lse is the natural-log logsumexp of the allowed scores of a row;
  R8  with packed documents the rotary positions are 0..S-1 along the batch row,
      or, when asked for (``rope_doc_positions``), the token's offset inside its
      document, so that each packed document is rotated as if it stood alone;
  R22 the FP8 forward takes q, k, v as E4M3 codes with one scale per tensor, q
      and k already rotated; its exact result is attention over the decoded
      values times their scales.

Pins (tests that fix this oracle to something other than itself) live in
``tests/test_oracle_pins.py``: torch's float64 scaled_dot_product_attention and
autograd as a library special case, central finite differences, the complex
multiplication form of the rotation, closed forms (S=1, q=0 prefix means, the
ALiBi geometric mean, v constant), invariants (rows of P sum to 1, rotation
preserves norms, relative-position property, gradient sums per document) and
the page's 20B head layout.  R1, R2 and R5 are readings the pages do not fix:
the tests pin the oracle to them, not to the pages ("parity unpinned" against
the pages for the rotation convention and the slope schedule).
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Rotary position embedding
# --------------------------------------------------------------------------

def rope_inv_freq(rotary_dim: int, base: float) -> np.ndarray:
    """Frequencies base^(-2p / rotary_dim) for p = 0 .. rotary_dim/2 - 1 (R3)."""
    if rotary_dim % 2:
        raise ValueError("rotary_dim must be even")
    p = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * p / rotary_dim)


def rope_angles(positions: np.ndarray, rotary_dim: int, base: float) -> np.ndarray:
    """theta[t, p] = positions[t] * inv_freq[p]  (shape [len(positions), rd/2])."""
    pos = np.asarray(positions, dtype=np.float64)
    return np.multiply.outer(pos, rope_inv_freq(rotary_dim, base))


def rope_rotate(x: np.ndarray, positions: np.ndarray, rotary_dim: int, base: float,
                inverse: bool = False) -> np.ndarray:
    """NeoX rotate-half rotation of the first ``rotary_dim`` dims of x (R1, R2).

    ``x`` is [..., S, D] and ``positions`` has length S.  With ``inverse`` the
    rotation is by -theta (the transpose R^T), which maps a gradient with
    respect to the rotated vector back to the unrotated one.  Dims at or beyond
    ``rotary_dim`` pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    rd = int(rotary_dim)
    if rd == 0:
        return x.copy()
    half = rd // 2
    theta = rope_angles(positions, rd, base)
    if inverse:
        theta = -theta
    c = np.cos(theta)
    s = np.sin(theta)
    x1 = x[..., :half]
    x2 = x[..., half:rd]
    y = x.copy()
    y[..., :half] = x1 * c - x2 * s
    y[..., half:rd] = x2 * c + x1 * s
    return y


# --------------------------------------------------------------------------
# Masks and biases
# --------------------------------------------------------------------------

def alibi_slopes(H: int) -> np.ndarray:
    """Slope of head h: 2^(-8 (h+1) / H), h = 0 .. H-1 (R5)."""
    h = np.arange(H, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / H)


def doc_index(offsets_row: Optional[np.ndarray], S: int) -> np.ndarray:
    """doc(t) for t = 0..S-1: the d with offsets[d] <= t < offsets[d+1].

    ``offsets_row`` starts at 0, never decreases and ends at S; empty documents
    (equal neighbours) own no token.  None means a single document.
    """
    if offsets_row is None:
        return np.zeros(S, dtype=np.int64)
    off = np.asarray(offsets_row, dtype=np.int64)
    t = np.arange(S)
    # number of offsets <= t, minus one: the last d with offsets[d] <= t
    return np.searchsorted(off, t, side="right") - 1


def rope_positions(S: int, offsets_row: Optional[np.ndarray] = None,
                   per_document: bool = False) -> np.ndarray:
    """Rotary position of each token of a batch row (R3, R8): t, or with
    ``per_document`` the offset t - offsets[doc(t)] of t inside its document."""
    t = np.arange(S)
    if not per_document or offsets_row is None:
        return t
    off = np.asarray(offsets_row, dtype=np.int64)
    return t - off[doc_index(offsets_row, S)]


def allowed_mask(S: int, causal: bool, offsets_row: Optional[np.ndarray]) -> np.ndarray:
    """Boolean [S, S]: allowed[i, j] (R6)."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    ok = np.ones((S, S), dtype=bool)
    if causal:
        ok &= j <= i
    d = doc_index(offsets_row, S)
    ok &= d[:, None] == d[None, :]
    return ok


def alibi_bias(S: int, slope: float) -> np.ndarray:
    """bias[i, j] = -slope * (i - j)  (R4)."""
    i = np.arange(S, dtype=np.float64)[:, None]
    j = np.arange(S, dtype=np.float64)[None, :]
    return -float(slope) * (i - j)


# --------------------------------------------------------------------------
# One head: forward and backward by the definition
# --------------------------------------------------------------------------

def _head_probs(qr, kr, scale, bias, allowed):
    """Scores of one head, then P = exp(s - lse) row by row (two passes)."""
    s = scale * (qr @ kr.T)
    if bias is not None:
        s += bias
    s[~allowed] = -np.inf
    m = s.max(axis=1)                       # row max over allowed keys
    s -= m[:, None]
    np.exp(s, out=s)                        # masked entries become exactly 0
    l = s.sum(axis=1)
    lse = m + np.log(l)
    s /= l[:, None]                         # s now holds P
    return s, lse


def head_forward(q, k, v, *, rotary_dim, rope_base, causal, scale, slope=None,
                 offsets_row=None, positions=None):
    """o [S, D] and lse [S] of one head; ``positions`` are the rotary positions
    (default 0..S-1)."""
    S = q.shape[0]
    pos = np.arange(S) if positions is None else np.asarray(positions)
    qr = rope_rotate(q, pos, rotary_dim, rope_base)
    kr = rope_rotate(k, pos, rotary_dim, rope_base)
    bias = alibi_bias(S, slope) if slope is not None else None
    P, lse = _head_probs(qr, kr, scale, bias, allowed_mask(S, causal, offsets_row))
    o = P @ v
    return o, lse


def head_backward(q, k, v, dout, *, rotary_dim, rope_base, causal, scale, slope=None,
                  offsets_row=None, positions=None):
    """(o, lse, dq, dk, dv) of one head, by differentiating the definition.

    dv_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;  Delta_i = dO_i . o_i;
    dS_ij = P_ij (dP_ij - Delta_i);  dq~_i = scale sum_j dS_ij k~_j;
    dk~_j = scale sum_i dS_ij q~_i;  dq = R^T dq~,  dk = R^T dk~.
    The bias does not depend on q, k, v, so it adds no gradient term.
    """
    S = q.shape[0]
    pos = np.arange(S) if positions is None else np.asarray(positions)
    qr = rope_rotate(q, pos, rotary_dim, rope_base)
    kr = rope_rotate(k, pos, rotary_dim, rope_base)
    bias = alibi_bias(S, slope) if slope is not None else None
    P, lse = _head_probs(qr, kr, scale, bias, allowed_mask(S, causal, offsets_row))
    o = P @ v
    dv = P.T @ dout
    dP = dout @ v.T
    delta = np.sum(dout * o, axis=1)
    dS = P * (dP - delta[:, None])
    dqr = scale * (dS @ kr)
    dkr = scale * (dS.T @ qr)
    dq = rope_rotate(dqr, pos, rotary_dim, rope_base, inverse=True)
    dk = rope_rotate(dkr, pos, rotary_dim, rope_base, inverse=True)
    return o, lse, dq, dk, dv


# --------------------------------------------------------------------------
# Batched front ends ([B, H, S, D] float64 arrays)
# --------------------------------------------------------------------------

def _heads(B: int, H: int, heads: Optional[Iterable[Tuple[int, int]]]):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [(int(b), int(h)) for b, h in heads]


def _slopes(H, alibi):
    if alibi is None or alibi is False:
        return None
    if alibi is True:
        return alibi_slopes(H)
    return np.asarray(alibi, dtype=np.float64)


def attn_fwd(q, k, v, *, rotary_dim: int, rope_base: float = 10000.0, causal: bool = True,
             softmax_scale: Optional[float] = None, alibi=False,
             doc_offsets: Optional[np.ndarray] = None,
             heads: Optional[Sequence[Tuple[int, int]]] = None,
             rope_doc_positions: bool = False):
    """Forward of attention over [B, H, S, D] float64 inputs.

    ``alibi`` is False, True (slopes by R5) or an explicit [H] slope array.
    ``rope_doc_positions`` restarts the rotary positions at each document (R8).
    ``heads`` restricts the work to a list of (b, h); the results are then
    stacked in that order as o [n, S, D] and lse [n, S].  Heads are independent,
    so a restricted run gives exactly the full run's values for those heads.
    """
    B, H, S, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    slopes = _slopes(H, alibi)
    hl = _heads(B, H, heads)
    o = np.empty((len(hl), S, D))
    lse = np.empty((len(hl), S))
    for n, (b, h) in enumerate(hl):
        offs = None if doc_offsets is None else doc_offsets[b]
        o[n], lse[n] = head_forward(
            q[b, h], k[b, h], v[b, h], rotary_dim=rotary_dim, rope_base=rope_base,
            causal=causal, scale=scale, slope=None if slopes is None else slopes[h],
            offsets_row=offs, positions=rope_positions(S, offs, rope_doc_positions))
    if heads is None:
        return o.reshape(B, H, S, D), lse.reshape(B, H, S)
    return o, lse


def attn_bwd(q, k, v, dout, *, rotary_dim: int, rope_base: float = 10000.0,
             causal: bool = True, softmax_scale: Optional[float] = None, alibi=False,
             doc_offsets: Optional[np.ndarray] = None,
             heads: Optional[Sequence[Tuple[int, int]]] = None,
             rope_doc_positions: bool = False):
    """(o, lse, dq, dk, dv) over [B, H, S, D] float64 inputs; see attn_fwd."""
    B, H, S, D = q.shape
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    slopes = _slopes(H, alibi)
    hl = _heads(B, H, heads)
    out = [np.empty((len(hl), S, D)), np.empty((len(hl), S)), np.empty((len(hl), S, D)),
           np.empty((len(hl), S, D)), np.empty((len(hl), S, D))]
    for n, (b, h) in enumerate(hl):
        offs = None if doc_offsets is None else doc_offsets[b]
        res = head_backward(
            q[b, h], k[b, h], v[b, h], dout[b, h], rotary_dim=rotary_dim,
            rope_base=rope_base, causal=causal, scale=scale,
            slope=None if slopes is None else slopes[h], offsets_row=offs,
            positions=rope_positions(S, offs, rope_doc_positions))
        for dst, r in zip(out, res):
            dst[n] = r
    if heads is None:
        return (out[0].reshape(B, H, S, D), out[1].reshape(B, H, S),
                out[2].reshape(B, H, S, D), out[3].reshape(B, H, S, D),
                out[4].reshape(B, H, S, D))
    return tuple(out)



# --------------------------------------------------------------------------
# Autoregressive decoding (one new token against a key/value cache)
# --------------------------------------------------------------------------

def attn_decode(q, k, v, k_cache, v_cache, *, rotary_dim: int, rope_base: float = 10000.0,
                softmax_scale: Optional[float] = None):
    """One decoding step of one head.

    The FasterTransformer GPT-NeoX guide ("FasterTransformer GPT-NeoX 推理指南",
    section "背景") separates the context decoder from a decoder that generates
    one token at a time against the earlier tokens.  Read plainly, one step is
    the last row of causal attention over the sequence so far: the new token
    sits at position t = len(k_cache); its query and key are rotated at that
    position (R1-R3); its rotated key and its value join the cache; its query
    attends over all t + 1 cached tokens.  The cache holds keys already rotated,
    each at its own position, as a decoder stores them.

    q, k, v: [D] float64, the new token's projections (not rotated).
    k_cache, v_cache: [t, D] float64 (rotated keys; values).
    Returns (o [D], lse, k_rot [D]): the output, the natural-log logsumexp of
    the t + 1 scores, and the rotated key appended to the cache.
    """
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    t = int(np.asarray(k_cache).shape[0])
    scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)
    pos = np.array([t])
    q_rot = rope_rotate(q[None, :], pos, rotary_dim, rope_base)[0]
    k_rot = rope_rotate(np.asarray(k, dtype=np.float64)[None, :], pos, rotary_dim, rope_base)[0]
    keys = np.concatenate([np.asarray(k_cache, dtype=np.float64).reshape(t, D), k_rot[None, :]])
    vals = np.concatenate([np.asarray(v_cache, dtype=np.float64).reshape(t, D),
                           np.asarray(v, dtype=np.float64)[None, :]])
    s = scale * (keys @ q_rot)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e / l) @ vals, m + np.log(l), k_rot


# --------------------------------------------------------------------------
# FP8 (E4M3) forward
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Values of FP8 E4M3 codes (the OCP 8-bit format with 1 sign bit, 4
    exponent bits of bias 7 and 3 mantissa bits; no infinities, the codes with
    all exponent and mantissa bits set are NaN): exponent field e > 0 gives
    (-1)^s 2^(e-7) (1 + m/8), e = 0 gives the subnormal (-1)^s 2^-6 (m/8).
    The pages name FP8 compute (Transformer Engine, "GPT-NeoX 开源训练框架深度解读",
    the TE Dockerfile) without fixing a format; E4M3 is the reading (R22)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    v = s * np.where(e > 0, normal, sub)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def attn_fwd_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, *,
                 causal: bool = True, softmax_scale: Optional[float] = None,
                 heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Forward of the FP8 variant: q, k, v given as E4M3 codes [B, H, S, D] with
    one scale per tensor (value = decoded code x scale); q and k are already
    rotated (the rotation is applied before quantisation, R22).  The exact
    result is attention over the dequantised tensors, which is what this
    returns (o, lse); the tolerance of an FP8 kernel against it comes from the
    rounding of the probabilities to E4M3 (R23)."""
    q = e4m3_decode(q8) * float(q_scale)
    k = e4m3_decode(k8) * float(k_scale)
    v = e4m3_decode(v8) * float(v_scale)
    D = q.shape[-1]
    return attn_fwd(q, k, v, rotary_dim=0, causal=causal,
                    softmax_scale=1.0 / np.sqrt(D) if softmax_scale is None else softmax_scale,
                    heads=heads)
