"""Seeded synthetic workloads for causal NeoX-rotary attention.

This module only *generates inputs*: shapes, seeded normal draws, rounding of
those draws to the storage type, and the packed-document layout.  It holds none
of the attention arithmetic, so the CPU oracle and the HIP path can both be fed
from it without sharing any of the method.

Shapes follow the GPT-NeoX pages:
  * context length 2048 ("GPT-NeoX: Как 20-миллиардная модель от EleutherAI
    изменила открытый ИИ", section "Ключевые особенности и архитектура");
  * the 20B head layout, 64 heads x 96 dims with 24 rotary dims
    ("FasterTransformer GPT-NeoX 推理指南", section "模型配置", config.ini fields
    head_num / size_per_head / rotary_embedding);
  * RoPE and ALiBi as the two position schemes ("GPT-NeoX 开源训练框架深度解读",
    section "架构创新").

Recipe (every workload): numpy ``SeedSequence(seed).spawn(5)`` gives independent
streams for q, k, v, dO and the document lengths; q, k, v, dO are N(0, 1) draws
in float64, multiplied by ``amp``, cast to float32 and, for bf16 (f16)
workloads, rounded to bfloat16 (IEEE half) with round-to-nearest-even.  Document lengths are drawn per
batch row from that row's own child stream.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
F16 = "f16"
F32 = "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: sizes, position scheme and input recipe."""

    name: str
    B: int
    H: int
    S: int
    D: int
    rotary_dim: int
    dtype: str  # "bf16", "f16" or "f32": storage type of q, k, v, o, dO
    backward: bool = True
    rope_base: float = 10000.0
    causal: bool = True
    alibi: bool = False
    packed_docs: bool = False
    doc_min: int = 64
    doc_max: int = 4096
    amp: float = 1.0
    seed: int = 20260000
    # With packed documents and RoPE: rotary positions restart at each document
    # start (each document rotated as if it stood alone).  Scores depend only on
    # position differences inside a document, so the attention results equal
    # those of positions 0..S-1 along the row; the flag tells the oracle which
    # reading to compute.
    rope_doc_positions: bool = False

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the library is measured and checked on, the S=2048, D=128
# shape used for the forward-efficiency figure and the packed documents with
# RoPE.  Seeds are 20260000 + the workload's index (1-based for the five, 6 for
# the D=128 shape, 7 for RoPE with documents).
WORKLOADS = {
    "fp32_s128_d64": Workload(
        "fp32_s128_d64", B=1, H=2, S=128, D=64, rotary_dim=64, dtype=F32,
        backward=False, seed=20260001),
    "bf16_s2048_d64_rd16": Workload(
        "bf16_s2048_d64_rd16", B=8, H=12, S=2048, D=64, rotary_dim=16,
        dtype=BF16, seed=20260002),
    "neox20b_s2048_h64_d96_rd24": Workload(
        "neox20b_s2048_h64_d96_rd24", B=4, H=64, S=2048, D=96, rotary_dim=24,
        dtype=BF16, seed=20260003),
    "long_s16384_d128": Workload(
        "long_s16384_d128", B=1, H=32, S=16384, D=128, rotary_dim=128,
        dtype=BF16, amp=0.5, seed=20260004),
    "alibi_docs_s4096_d128": Workload(
        "alibi_docs_s4096_d128", B=4, H=32, S=4096, D=128, rotary_dim=0,
        dtype=BF16, alibi=True, packed_docs=True, seed=20260005),
    "rope_s2048_d128": Workload(
        "rope_s2048_d128", B=4, H=32, S=2048, D=128, rotary_dim=128,
        dtype=BF16, seed=20260006),
    # The packed-document layout of the ALiBi workload with RoPE instead (a
    # quarter of the head dim rotated, the 20B model's 24 of 96), positions
    # restarting at each document.
    "rope_docs_s4096_d128": Workload(
        "rope_docs_s4096_d128", B=4, H=32, S=4096, D=128, rotary_dim=32,
        dtype=BF16, packed_docs=True, rope_doc_positions=True, seed=20260007),
}

# Workload whose fwd+bwd throughput is the headline figure: the 2048-token
# context with the 20B head layout.
BENCH_WORKLOAD = "neox20b_s2048_h64_d96_rd24"
# Shape for the causal-forward efficiency figure (S=2048, D=128).
FWD_TARGET_WORKLOAD = "rope_s2048_d128"


def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    NaN is not expected in generated data; infinities stay infinities.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (uint16 bits for bf16 / f16, float32 for f32) widened exactly."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    if dtype == F16:
        return np.asarray(arr, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(arr).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """Generated tensors of one workload.

    ``q, k, v, dout`` are the storage values: uint16 bit patterns for bf16 and
    f16 workloads, float32 for f32 workloads, shaped [B, H, S, D].  ``doc_offsets``
    is int32 [B, n_docs_max + 1] (0 first, S last, non-decreasing; rows with
    fewer documents repeat S), or None for one document per row.
    """

    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dout: Optional[np.ndarray]
    doc_offsets: Optional[np.ndarray]

    def as_f64(self, name: str) -> np.ndarray:
        """A generated tensor widened exactly to float64."""
        a = getattr(self, name)
        if a is None:
            return None
        return storage_to_f64(a, self.wl.dtype)


def pack_documents(rng: np.random.Generator, S: int, lo: int, hi: int) -> list:
    """Document lengths for one batch row: draws L ~ UniformInt[lo, hi]
    (inclusive) until the row is full; when the room left after a draw would be
    shorter than ``lo`` the draw is replaced by all the room left, so every
    length lies in [lo, hi] (or is S itself when S < lo) and they sum to S."""
    lengths = []
    remaining = S
    while remaining > 0:
        L = int(rng.integers(lo, hi + 1))
        if remaining - L < lo:
            L = remaining
        lengths.append(L)
        remaining -= L
    return lengths


def doc_offsets_from_lengths(rows: list, S: int) -> np.ndarray:
    """Per-row lengths -> int32 [B, n_max + 1] cumulative offsets padded with S."""
    n_max = max(len(r) for r in rows)
    out = np.full((len(rows), n_max + 1), S, dtype=np.int32)
    for b, lengths in enumerate(rows):
        out[b, 0] = 0
        out[b, 1:len(lengths) + 1] = np.cumsum(lengths)
    return out


def _draw(rng: np.random.Generator, shape, amp: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if amp != 1.0:
        x *= amp
    x32 = x.astype(np.float32)
    if dtype == BF16:
        return round_to_bf16_bits(x32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)  # round to nearest even
    return x32


def generate(wl: Workload, with_dout: Optional[bool] = None) -> Inputs:
    """Seeded inputs of ``wl`` (see the module docstring for the recipe)."""
    if with_dout is None:
        with_dout = wl.backward
    ss_q, ss_k, ss_v, ss_do, ss_docs = np.random.SeedSequence(wl.seed).spawn(5)
    shape = (wl.B, wl.H, wl.S, wl.D)
    q = _draw(np.random.default_rng(ss_q), shape, wl.amp, wl.dtype)
    k = _draw(np.random.default_rng(ss_k), shape, wl.amp, wl.dtype)
    v = _draw(np.random.default_rng(ss_v), shape, wl.amp, wl.dtype)
    dout = _draw(np.random.default_rng(ss_do), shape, wl.amp, wl.dtype) if with_dout else None
    docs = None
    if wl.packed_docs:
        rows = [pack_documents(np.random.default_rng(s), wl.S, wl.doc_min, wl.doc_max)
                for s in ss_docs.spawn(wl.B)]
        docs = doc_offsets_from_lengths(rows, wl.S)
    return Inputs(wl, q, k, v, dout, docs)



def allowed_pairs(S: int, causal: bool = True, doc_offsets_row=None) -> int:
    """Count of (query, key) pairs one head attends over: the unit of
    algorithmic work.  Causal: L(L+1)/2 per document of length L; otherwise L^2.
    """
    if doc_offsets_row is None:
        lengths = [S]
    else:
        off = np.asarray(doc_offsets_row, dtype=np.int64)
        lengths = [int(x) for x in np.diff(off) if x > 0]
    if causal:
        return sum(L * (L + 1) // 2 for L in lengths)
    return sum(L * L for L in lengths)


def total_pairs(inp: "Inputs") -> int:
    """Allowed pairs summed over all B x H heads of generated inputs."""
    wl = inp.wl
    if inp.doc_offsets is None:
        return wl.B * wl.H * allowed_pairs(wl.S, wl.causal)
    return wl.H * sum(allowed_pairs(wl.S, wl.causal, row) for row in inp.doc_offsets)


# ---------------------------------------------------------------- decoding


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decoding step for B sequences: the new token's q, k, v [B, H, D] and
    key/value caches [B, H, cap, D] holding ``lens[b]`` earlier tokens.

    Sizes follow the GPT-NeoX-20B inference configuration of the
    FasterTransformer guide ("FasterTransformer GPT-NeoX 推理指南", sections
    "模型配置" and "采样与解码参数": 64 heads of 96 dims, 24 rotary dims,
    request batch 8) with the 2048-token context of the model.
    ``lens``: "full" puts every sequence at position cap - 1 (the whole cache
    is read); "ragged" draws each row's position uniformly from [0, cap - 1].
    """

    name: str
    B: int
    H: int
    D: int
    rotary_dim: int
    cap: int
    dtype: str
    lens: str = "full"
    rope_base: float = 10000.0
    seed: int = 20260100

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def with_sizes(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS = {
    "neox20b_decode_b8_cap2048": DecodeWorkload(
        "neox20b_decode_b8_cap2048", B=8, H=64, D=96, rotary_dim=24, cap=2048, dtype=BF16,
        lens="full", seed=20260101),
    "neox20b_decode_b8_cap2048_ragged": DecodeWorkload(
        "neox20b_decode_b8_cap2048_ragged", B=8, H=64, D=96, rotary_dim=24, cap=2048,
        dtype=BF16, lens="ragged", seed=20260102),
}
DECODE_BENCH_WORKLOAD = "neox20b_decode_b8_cap2048"


@dataclasses.dataclass
class DecodeInputs:
    """Generated decode inputs: ``q, k, v`` [B, H, D] and ``k_cache, v_cache``
    [B, H, cap, D] as storage values (uint16 bf16 bits or float32), ``lens``
    int32 [B].  Cache rows hold N(0, 1) draws: any vector is a valid rotated
    key, so the cache needs no rotation to be generated."""

    wl: DecodeWorkload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    lens: np.ndarray

    def as_f64(self, name: str) -> np.ndarray:
        return storage_to_f64(getattr(self, name), self.wl.dtype)


def generate_decode(wl: DecodeWorkload) -> DecodeInputs:
    """Seeded decode inputs: ``SeedSequence(seed).spawn(6)`` streams for q, k, v,
    the key cache, the value cache and the lengths; N(0, 1) draws rounded to the
    storage type as for ``generate``."""
    ss = np.random.SeedSequence(wl.seed).spawn(6)
    tok = (wl.B, wl.H, wl.D)
    cache = (wl.B, wl.H, wl.cap, wl.D)
    q, k, v = (_draw(np.random.default_rng(s), tok, 1.0, wl.dtype) for s in ss[:3])
    kc = _draw(np.random.default_rng(ss[3]), cache, 1.0, wl.dtype)
    vc = _draw(np.random.default_rng(ss[4]), cache, 1.0, wl.dtype)
    if wl.lens == "full":
        lens = np.full(wl.B, wl.cap - 1, dtype=np.int32)
    elif wl.lens == "ragged":
        lens = np.random.default_rng(ss[5]).integers(0, wl.cap, size=wl.B).astype(np.int32)
    else:
        raise ValueError(f"unknown lens mode {wl.lens!r}")
    return DecodeInputs(wl, q, k, v, kc, vc, lens)


def decode_bytes(wl: DecodeWorkload, lens) -> int:
    """Algorithmic HBM bytes of one decoding step: every (b, h) reads the t + 1
    cached key and value rows it attends over (the new row included) once;
    the new token's q, k, v are read, its key and value written into the
    cache, and o and the fp32 lse written."""
    es = 4 if wl.dtype == F32 else 2
    rows = sum(int(t) + 1 for t in lens) * wl.H
    return rows * 2 * wl.D * es + wl.B * wl.H * (6 * wl.D * es + 4)


# ---------------------------------------------------------------- FP8 (E4M3)

def _e4m3_table() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0..126: code = (e << 3) | m
    is 2^(e-7) (1 + m/8) for e > 0 and 2^-6 m/8 for e = 0 (OCP FP8 E4M3)."""
    code = np.arange(127)
    e, m = code >> 3, code & 7
    return np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes (uint8), round to nearest, ties to the even code,
    saturating at +-448 (no NaN produced for finite inputs)."""
    x = np.asarray(x, dtype=np.float64)
    table = _e4m3_table()
    a = np.minimum(np.abs(x), table[-1])
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, 126)
    lo = hi - 1
    dlo, dhi = a - table[lo], table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a <= 0, 0, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """FP8 forward problem: q~, k~ (already rotated) and v drawn N(0, 1), each
    quantised to E4M3 with one scale per tensor, scale = amax / 448 (the
    largest value maps to the largest code)."""

    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool = True
    seed: int = 20260200

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


@dataclasses.dataclass
class Fp8Inputs:
    wl: Fp8Workload
    q8: np.ndarray  # uint8 E4M3 codes [B, H, S, D]
    k8: np.ndarray
    v8: np.ndarray
    scales: tuple   # (q, k, v)


FP8_WORKLOADS = {
    "fp8_s2048_d128": Fp8Workload("fp8_s2048_d128", B=4, H=32, S=2048, D=128, seed=20260201),
    "fp8_neox20b_s2048_d96": Fp8Workload("fp8_neox20b_s2048_d96", B=4, H=64, S=2048, D=96,
                                         seed=20260202),
}
FP8_BENCH_WORKLOAD = "fp8_s2048_d128"


def generate_fp8(wl: Fp8Workload) -> Fp8Inputs:
    """Seeded FP8 inputs: ``SeedSequence(seed).spawn(3)`` streams for q, k, v."""
    out, scales = [], []
    for s in np.random.SeedSequence(wl.seed).spawn(3):
        x = np.random.default_rng(s).standard_normal((wl.B, wl.H, wl.S, wl.D))
        scale = float(np.abs(x).max()) / 448.0
        out.append(e4m3_encode(x / scale))
        scales.append(scale)
    return Fp8Inputs(wl, out[0], out[1], out[2], tuple(scales))
