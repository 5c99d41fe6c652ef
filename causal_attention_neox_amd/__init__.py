"""causal_attention_neox_amd: causal multi-head attention with GPT-NeoX rotary
position embedding for AMD MI355X (gfx950).

The compute lives in ``libneoxattn.so`` (hand-written HIP kernels behind the C
ABI of ``include/neoxattn.h``).  This package is its thin Python binding: the
functions below carry the C names, take torch tensors that already live on
the GPU, and only marshal pointers, sizes and the current stream.  PyTorch
supplies device memory and streams; no step of the attention runs in it.

The compute calls allocate nothing: a RoPE call with rotary_dim > 0 needs the
rotary table prepared first with ``neox_rope_table_prepare(max_S, rotary_dim,
rope_base)`` (else NeoxError with NEOX_E_NOT_PREPARED).  ``attention()`` wraps
the forward and backward calls in a torch autograd Function and prepares the
table itself.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import _lib
from ._lib import (NEOX_BF16, NEOX_F16, NEOX_F32, NEOX_OUT_F32, NEOX_OUT_SAME, NEOX_POS_ALIBI,
                   NEOX_POS_NONE, NEOX_POS_ROPE)

__all__ = [
    "NeoxError", "neox_status_str", "neox_rope_attn_fwd", "neox_rope_attn_bwd",
    "neox_rope_attn_fwd_workspace_size", "neox_rope_attn_bwd_workspace_size",
    "neox_attn_fwd_ex", "neox_attn_bwd_ex",
    "neox_rope_attn_decode_workspace_size", "neox_rope_attn_decode",
    "neox_rope_attn_decode_noalloc", "neox_attn_fwd_fp8",
    "neox_check_doc_offsets", "neox_rope_table_prepare", "neox_attn_plan", "attention",
    "NEOX_F32", "NEOX_BF16", "NEOX_F16", "NEOX_POS_NONE", "NEOX_POS_ROPE", "NEOX_POS_ALIBI",
    "NEOX_OUT_SAME", "NEOX_OUT_F32",
]


class NeoxError(RuntimeError):
    """A non-zero status returned by libneoxattn."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {neox_status_str(status)} (status {status})")


def neox_status_str(status: int) -> str:
    return _lib.load().neox_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise NeoxError(status, where)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return NEOX_BF16
    if t.dtype == torch.float16:
        return NEOX_F16
    if t.dtype == torch.float32:
        return NEOX_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16, torch.float16 or "
                    "torch.float32")


def _shape(q):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, S, D]")
    return tuple(int(x) for x in q.shape)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def neox_rope_attn_fwd_workspace_size(B: int, H: int, S: int, D: int) -> int:
    return int(_lib.load().neox_rope_attn_fwd_workspace_size(B, H, S, D))


def neox_rope_attn_fwd(q, k, v, o, lse, rotary_dim: int, rope_base: float = 10000.0,
                       causal: bool = True, softmax_scale: Optional[float] = None,
                       workspace=None, stream=None) -> None:
    """Calls neox_rope_attn_fwd on contiguous [B, H, S, D] tensors (o, lse written).
    ``workspace`` is None or a uint8 device tensor of at least
    neox_rope_attn_fwd_workspace_size() bytes (pre-rotated queries and keys)."""
    B, H, S, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().neox_rope_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, int(rotary_dim),
        float(rope_base), int(bool(causal)), scale, _dtype_code(q), _ptr(workspace),
        _nbytes(workspace), _stream(stream))
    _check(st, "neox_rope_attn_fwd")


def neox_rope_attn_bwd_workspace_size(B: int, H: int, S: int, D: int) -> int:
    return int(_lib.load().neox_rope_attn_bwd_workspace_size(B, H, S, D))


def neox_rope_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, rotary_dim: int,
                       rope_base: float = 10000.0, causal: bool = True,
                       softmax_scale: Optional[float] = None, workspace=None,
                       stream=None) -> None:
    """Calls neox_rope_attn_bwd on contiguous tensors (dq, dk, dv written).
    ``workspace`` is a uint8 device tensor of at least the queried size."""
    B, H, S, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    nbytes = _nbytes(workspace)
    st = _lib.load().neox_rope_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, S, D, int(rotary_dim), float(rope_base), int(bool(causal)), scale, _dtype_code(q),
        _ptr(workspace), nbytes, _stream(stream))
    _check(st, "neox_rope_attn_bwd")


def _event_array(events):
    """hipEvent_t handles of torch.cuda.Event objects (or raw ints) as a void* array.
    A torch event exists only after its first record(); record it once before."""
    if events is None:
        return None
    handles = [e if isinstance(e, int) else int(e.cuda_event) for e in events]
    if any(h == 0 for h in handles):
        raise ValueError("phase events must be created (recorded once) before use")
    return (ctypes.c_void_p * len(handles))(*handles)


def _make_args(q, *, pos, rotary_dim, rope_base, alibi_slopes, causal, softmax_scale,
               doc_offsets, out_f32, tensors, phase_events=None, reuse_rotated_qk=False):
    B, H, S, D = _shape(q)
    a = _lib.NeoxAttnArgs()
    a.B, a.H, a.S, a.D = B, H, S, D
    a.dtype = _dtype_code(q)
    a.pos = int(pos)
    a.rotary_dim = int(rotary_dim)
    a.rope_base = float(rope_base)
    a.alibi_slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    a.causal = int(bool(causal))
    a.softmax_scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if doc_offsets is not None:
        a.doc_offsets = doc_offsets.data_ptr()
        a.n_docs = int(doc_offsets.shape[1]) - 1
    a.out_dtype = NEOX_OUT_F32 if out_f32 else NEOX_OUT_SAME
    a.reuse_rotated_qk = int(bool(reuse_rotated_qk))
    strides = (_lib.NeoxStrides * 8)()
    for n, t in enumerate(tensors):
        if t is not None:
            if t.stride(3) != 1:
                raise ValueError("the head dim must be contiguous")
            strides[n] = _lib.NeoxStrides(t.stride(0), t.stride(1), t.stride(2))
    a.strides = ctypes.cast(strides, ctypes.POINTER(_lib.NeoxStrides))
    ev = _event_array(phase_events)
    if ev is not None:
        a.phase_events = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    return a, (strides, ev)


def neox_attn_fwd_ex(q, k, v, o, lse, *, pos: int = NEOX_POS_ROPE, rotary_dim: int = 0,
                     rope_base: float = 10000.0, alibi_slopes=None, causal: bool = True,
                     softmax_scale: Optional[float] = None, doc_offsets=None,
                     out_f32: bool = False, workspace=None, phase_events=None,
                     stream=None) -> None:
    """Calls neox_attn_fwd_ex; strides are taken from the tensors.
    ``doc_offsets`` is an int32 device tensor [B, n_docs + 1]; ``workspace`` as
    for neox_rope_attn_fwd; ``phase_events`` is None or 3 events (before the
    call, after the q/k rotation pass, after the attention kernel)."""
    a, keep = _make_args(q, pos=pos, rotary_dim=rotary_dim, rope_base=rope_base,
                         alibi_slopes=alibi_slopes, causal=causal, softmax_scale=softmax_scale,
                         doc_offsets=doc_offsets, out_f32=out_f32,
                         tensors=[q, k, v, o, None, None, None, None],
                         phase_events=phase_events)
    st = _lib.load().neox_attn_fwd_ex(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(lse), _ptr(workspace), _nbytes(workspace),
                                      _stream(stream))
    del keep
    _check(st, "neox_attn_fwd_ex")


def neox_attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, *, pos: int = NEOX_POS_ROPE,
                     rotary_dim: int = 0, rope_base: float = 10000.0, alibi_slopes=None,
                     causal: bool = True, softmax_scale: Optional[float] = None,
                     doc_offsets=None, out_f32: bool = False, workspace=None,
                     phase_events=None, reuse_rotated_qk: bool = False, stream=None) -> None:
    """Calls neox_attn_bwd_ex; strides are taken from the tensors.  ``phase_events``
    is None or 4 events (before/after the preprocess, after the dQ kernel --
    the fp32 path: after its main kernels --, at the end).  ``reuse_rotated_qk``: the workspace was the
    forward's workspace and still holds the rotated q and k."""
    a, keep = _make_args(q, pos=pos, rotary_dim=rotary_dim, rope_base=rope_base,
                         alibi_slopes=alibi_slopes, causal=causal, softmax_scale=softmax_scale,
                         doc_offsets=doc_offsets, out_f32=out_f32,
                         tensors=[q, k, v, o, dout, dq, dk, dv], phase_events=phase_events,
                         reuse_rotated_qk=reuse_rotated_qk)
    nbytes = _nbytes(workspace)
    st = _lib.load().neox_attn_bwd_ex(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(workspace), nbytes, _stream(stream))
    del keep
    _check(st, "neox_attn_bwd_ex")


def neox_rope_attn_decode_workspace_size(B: int, H: int, D: int, cap: int) -> int:
    return int(_lib.load().neox_rope_attn_decode_workspace_size(B, H, D, cap))


def neox_rope_attn_decode(q, k, v, k_cache, v_cache, cache_lens, o, lse, rotary_dim: int,
                          rope_base: float = 10000.0, softmax_scale: Optional[float] = None,
                          workspace=None, stream=None) -> None:
    """Calls neox_rope_attn_decode: q, k, v, o are [B, H, D]; k_cache, v_cache are
    [B, H, cap, D] (row cache_lens[b] is written); cache_lens is an int32 device
    tensor [B]; lse is fp32 [B, H]; ``workspace`` is a uint8 device tensor of at
    least neox_rope_attn_decode_workspace_size() bytes."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, D] and the caches [B, H, cap, D]")
    B, H, D = (int(x) for x in q.shape)
    cap = int(k_cache.shape[2])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().neox_rope_attn_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), _ptr(o),
        _ptr(lse), B, H, D, cap, int(rotary_dim), float(rope_base), scale, _dtype_code(q),
        _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "neox_rope_attn_decode")


def neox_rope_attn_decode_noalloc(q, k, v, k_cache, v_cache, cache_lens, o, lse,
                                  rotary_dim: int, rope_base: float = 10000.0,
                                  softmax_scale: Optional[float] = None, stream=None) -> None:
    """Calls neox_rope_attn_decode_noalloc: as neox_rope_attn_decode, with the
    chunk partials in the library's fixed per-device array instead of a
    workspace (calls on one device must not overlap)."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, D] and the caches [B, H, cap, D]")
    B, H, D = (int(x) for x in q.shape)
    cap = int(k_cache.shape[2])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().neox_rope_attn_decode_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), _ptr(o),
        _ptr(lse), B, H, D, cap, int(rotary_dim), float(rope_base), scale, _dtype_code(q),
        _stream(stream))
    _check(st, "neox_rope_attn_decode_noalloc")


def neox_attn_fwd_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, o, lse,
                      causal: bool = True, softmax_scale: Optional[float] = None,
                      stream=None) -> None:
    """Calls neox_attn_fwd_fp8: q8, k8, v8 are [B, H, S, D] tensors of E4M3 codes
    (uint8 or torch.float8_e4m3fn), q8 and k8 already rotated; o is bf16 or fp32
    [B, H, S, D]; lse is fp32 [B, H, S]."""
    import torch
    B, H, S, D = _shape(q8)
    if o.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("o must be bfloat16 or float32")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().neox_attn_fwd_fp8(
        _ptr(q8), _ptr(k8), _ptr(v8), float(q_scale), float(k_scale), float(v_scale), _ptr(o),
        _ptr(lse), B, H, S, D, int(bool(causal)), scale,
        NEOX_OUT_F32 if o.dtype == torch.float32 else NEOX_OUT_SAME, _stream(stream))
    _check(st, "neox_attn_fwd_fp8")


def neox_check_doc_offsets(offsets_host, S: int) -> int:
    """Status of neox_check_doc_offsets on a host int32 array [B, n_docs + 1]."""
    import numpy as np
    arr = np.ascontiguousarray(offsets_host, dtype=np.int32)
    B, n1 = arr.shape
    return int(_lib.load().neox_check_doc_offsets(arr.ctypes.data_as(ctypes.c_void_p), B,
                                                  n1 - 1, int(S)))


def neox_attn_plan(q, *, pos: int = NEOX_POS_ROPE, rotary_dim: int = 0, alibi_slopes=None,
                   doc_offsets=None, causal: bool = True, fwd_workspace: bool = True,
                   reuse_rotated_qk: bool = False) -> dict:
    """Calls neox_attn_plan for a call on tensors shaped and typed like q: the
    kernel forms the forward and the backward would launch (no device work)."""
    a, keep = _make_args(q, pos=pos, rotary_dim=rotary_dim, rope_base=10000.0,
                         alibi_slopes=alibi_slopes, causal=causal, softmax_scale=None,
                         doc_offsets=doc_offsets, out_f32=False, tensors=[None] * 8,
                         reuse_rotated_qk=reuse_rotated_qk)
    plan = _lib.NeoxPlan()
    st = _lib.load().neox_attn_plan(ctypes.byref(a), int(bool(fwd_workspace)), ctypes.byref(plan))
    del keep
    _check(st, "neox_attn_plan")
    return {name: int(getattr(plan, name)) for name, _ in _lib.NeoxPlan._fields_}


def neox_rope_table_prepare(max_S: int, rotary_dim: int, rope_base: float = 10000.0) -> None:
    """Set-up call: builds the rotary table of the current device for positions
    0..max_S-1 (allocates and waits; not under stream capture)."""
    _check(_lib.load().neox_rope_table_prepare(int(max_S), int(rotary_dim), float(rope_base)),
           "neox_rope_table_prepare")


def attention(q, k, v, rotary_dim: int = 0, rope_base: float = 10000.0, causal: bool = True,
              softmax_scale: Optional[float] = None, alibi: bool = False, alibi_slopes=None,
              doc_offsets=None, out_f32: bool = False):
    """Differentiable attention: o = attention(q, k, v); gradients flow to q, k, v.

    ``alibi=True`` switches from RoPE to ALiBi (then rotary_dim must be 0).
    """
    from ._autograd import NeoxAttentionFn
    return NeoxAttentionFn.apply(q, k, v, int(rotary_dim), float(rope_base), bool(causal),
                                 softmax_scale, bool(alibi), alibi_slopes, doc_offsets,
                                 bool(out_f32))
