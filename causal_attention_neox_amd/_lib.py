"""ctypes loader of libneoxattn.so with the C signatures of include/neoxattn.h.

The library is loaded on first use.  When it is missing the loader raises; no
other implementation stands in for it.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libneoxattn.so")

NEOX_OK = 0
NEOX_E_ARG = -1
NEOX_E_UNSUPPORTED = -2
NEOX_E_ALIGN = -3
NEOX_E_WORKSPACE = -4
NEOX_E_LAUNCH = -5
NEOX_E_DEVICE = -6
NEOX_E_ALLOC = -7
NEOX_E_NOT_PREPARED = -8
NEOX_E_TOO_LARGE = -9
NEOX_DECODE_SCRATCH_BYTES = 8 << 20

NEOX_F32 = 0
NEOX_BF16 = 1
NEOX_F16 = 2
NEOX_POS_NONE = 0
NEOX_POS_ROPE = 1
NEOX_POS_ALIBI = 2
NEOX_OUT_SAME = 0
NEOX_OUT_F32 = 1

# Every function the header declares, with (restype, argtypes).
c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class NeoxStrides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("seq", ctypes.c_int64)]


class NeoxAttnArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int), ("H", c_int), ("S", c_int), ("D", c_int),
        ("dtype", c_int), ("pos", c_int), ("rotary_dim", c_int), ("rope_base", c_float),
        ("alibi_slopes", c_void_p), ("causal", c_int), ("softmax_scale", c_float),
        ("doc_offsets", c_void_p), ("n_docs", c_int), ("out_dtype", c_int),
        ("strides", ctypes.POINTER(NeoxStrides)),
        ("phase_events", ctypes.POINTER(c_void_p)),
        ("reuse_rotated_qk", c_int),
    ]


class NeoxPlan(ctypes.Structure):
    _fields_ = [("fp32_path", c_int), ("fwd_rotation_pass", c_int), ("fwd_k_staging", c_int),
                ("fwd_rotate_q", c_int), ("alibi", c_int), ("bwd_rotation_pass", c_int)]


SIGNATURES = {
    "neox_status_str": (ctypes.c_char_p, [c_int]),
    "neox_rope_attn_fwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "neox_rope_attn_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_float,
                                   c_int, c_void_p, c_size_t, c_void_p]),
    "neox_rope_attn_bwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "neox_rope_attn_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p,
                                   c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_float,
                                   c_int, c_void_p, c_size_t, c_void_p]),
    "neox_attn_fwd_ex": (c_int, [ctypes.POINTER(NeoxAttnArgs), c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "neox_attn_bwd_ex": (c_int, [ctypes.POINTER(NeoxAttnArgs), c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "neox_rope_attn_decode_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "neox_rope_attn_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p,
                                      c_int, c_int, c_int, c_int, c_int, c_float, c_float,
                                      c_int, c_void_p, c_size_t, c_void_p]),
    "neox_rope_attn_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p,
                                              c_int, c_int, c_int, c_int, c_int, c_float,
                                              c_float, c_int, c_void_p]),
    "neox_attn_fwd_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_float, c_float, c_float,
                                  c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                  c_float, c_int, c_void_p]),
    "neox_check_doc_offsets": (c_int, [c_void_p, c_int, c_int, c_int]),
    "neox_rope_table_prepare": (c_int, [c_int, c_int, c_float]),
    "neox_attn_plan": (c_int, [ctypes.POINTER(NeoxAttnArgs), c_int, ctypes.POINTER(NeoxPlan)]),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """The loaded library; raises RuntimeError when it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m causal_attention_neox_amd.build` "
                    "(or __graft_entry__.build()); there is no fallback implementation")
            # One HIP runtime per process: torch's HIP libraries ask for the
            # runtime as libamdhip64.so while this library asks for
            # libamdhip64.so.7, so whichever loads first decides; loaded before
            # torch, this library would pull in a second runtime next to
            # torch's, and the one initialised second finds no device.  Loading
            # torch first makes both share torch's runtime.
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib
