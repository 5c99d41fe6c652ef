"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments before touching any device.

Only validation paths are called here (fake, never dereferenced pointers); no
call that would launch a kernel runs without a GPU.
"""

import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

from causal_attention_neox_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_ARG, E_UNSUP, E_ALIGN, E_WS, E_LAUNCH, E_DEV, E_ALLOC = 0, -1, -2, -3, -4, -5, -6, -7
E_NOT_PREPARED = -8
F32, BF16 = 0, 1
P = ctypes.c_void_p
A1, A2, A3, A4, A5, A6, A7, A8, A9 = (P(0x10000 * n) for n in range(1, 10))  # 16-byte aligned


@pytest.fixture(scope="session")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from causal_attention_neox_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(neox_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ("neox_rope_attn_fwd", "neox_rope_attn_bwd", "neox_rope_attn_bwd_workspace_size",
              "neox_rope_attn_fwd_workspace_size", "neox_attn_fwd_ex", "neox_attn_bwd_ex",
              "neox_rope_attn_decode", "neox_rope_attn_decode_workspace_size",
              "neox_status_str"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must cover the header"


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (neox_\w+)", out))
    missing = set(declared_functions()) - exported
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in (OK, E_ARG, E_UNSUP, E_ALIGN, E_WS, E_LAUNCH, E_DEV, E_ALLOC, E_NOT_PREPARED):
        assert lib.neox_status_str(s) != b"unknown status"
    assert b"neox_rope_table_prepare" in lib.neox_status_str(E_NOT_PREPARED)
    assert lib.neox_status_str(OK) == b"ok"
    assert lib.neox_status_str(12345) == b"unknown status"


def fwd(lib, q=A1, k=A2, v=A3, o=A4, lse=A5, B=2, H=4, S=128, D=64, rd=16, base=1e4, causal=1,
        scale=0.125, dtype=BF16, ws=None, wsb=0):
    return lib.neox_rope_attn_fwd(q, k, v, o, lse, B, H, S, D, rd, base, causal, scale, dtype,
                                  ws, wsb, None)


def bwd(lib, ws=None, wsb=None, dq=A7, B=2, H=4, S=128, D=64, rd=16, dtype=BF16, **kw):
    need = lib.neox_rope_attn_bwd_workspace_size(B, H, S, D)
    ws = P(0x100000) if ws is None else ws
    wsb = need if wsb is None else wsb
    return lib.neox_rope_attn_bwd(kw.get("q", A1), A2, A3, A4, A5, A6, dq, A8, A9, B, H, S, D,
                                  rd, 1e4, 1, 0.125, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_ARG), (dict(lse=None), E_ARG), (dict(B=0), E_ARG), (dict(H=-1), E_ARG),
    (dict(S=0), E_ARG), (dict(D=0), E_ARG), (dict(D=80), E_UNSUP), (dict(D=256), E_UNSUP),
    (dict(rd=15), E_ARG), (dict(rd=66), E_ARG), (dict(rd=-2), E_ARG),
    (dict(base=0.0), E_ARG), (dict(base=float("inf")), E_ARG), (dict(base=float("nan")), E_ARG),
    (dict(scale=0.0), E_ARG), (dict(scale=-1.0), E_ARG), (dict(scale=float("nan")), E_ARG),
    (dict(dtype=7), E_ARG), (dict(q=P(0x10002)), E_ALIGN), (dict(o=P(0x10008)), E_ALIGN),
    (dict(lse=P(0x10004)), E_ALIGN), (dict(B=1 << 16, H=1 << 8, S=1 << 8), E_ARG),
])
def test_forward_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_forward_workspace_validation(lib):
    """The forward workspace is optional; when given it must be large enough
    and 256-byte aligned (checked before any device work)."""
    need = lib.neox_rope_attn_fwd_workspace_size(2, 4, 128, 64)
    assert need == 2 * (2 * 4 * 128 * 64 * 2)  # rotated q and k, bf16
    assert fwd(lib, ws=P(0x100000), wsb=need - 1) == E_WS
    assert fwd(lib, ws=P(0x100010), wsb=need) == E_ALIGN
    if not os.path.exists("/dev/kfd"):
        assert fwd(lib, ws=P(0x100000), wsb=need) == E_DEV
        assert fwd(lib, ws=None, wsb=0) == E_DEV
    assert lib.neox_rope_attn_fwd_workspace_size(0, 1, 1, 64) == 0
    assert lib.neox_rope_attn_fwd_workspace_size(1 << 16, 1 << 8, 1 << 8, 64) == 0
    assert lib.neox_rope_attn_fwd_workspace_size(1, 1, 3, 96) == 2 * 768  # 576 rounded up, x2


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None, wsb=0), E_WS), (dict(ws=P(0)), E_WS), (dict(ws=P(0x100010)), E_ALIGN),
    (dict(dq=A1), E_ARG), (dict(dq=None), E_ARG), (dict(D=80), E_UNSUP), (dict(rd=3), E_ARG),
])
def test_backward_validation(lib, kw, status):
    if kw.get("wsb") == 0:
        assert bwd(lib, wsb=1) == E_WS
        return
    assert bwd(lib, **kw) == status


def make_args(**kw):
    a = _lib.NeoxAttnArgs()
    a.B, a.H, a.S, a.D = 2, 4, 128, 64
    a.dtype, a.pos, a.rotary_dim, a.rope_base = BF16, 1, 16, 1e4
    a.causal, a.softmax_scale, a.out_dtype = 1, 0.125, 0
    for n, v in kw.items():
        setattr(a, n, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(pos=9), E_ARG), (dict(pos=2), E_ARG),  # ALiBi with rotary_dim != 0
    (dict(pos=0), E_ARG), (dict(out_dtype=3), E_ARG),
    (dict(pos=2, rotary_dim=0, alibi_slopes=0x1002), E_ALIGN),
    (dict(pos=1, alibi_slopes=0x1000), E_ARG),  # slopes without ALiBi
    (dict(n_docs=3), E_ARG),                      # n_docs without offsets
    (dict(doc_offsets=0x1000, n_docs=0), E_ARG),
    (dict(doc_offsets=0x1002, n_docs=2), E_ALIGN),
    (dict(reuse_rotated_qk=2), E_ARG),
])
def test_ex_validation(lib, kw, status):
    a = make_args(**kw)
    assert lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None) == status


def test_ex_strides_validation(lib):
    strides = (_lib.NeoxStrides * 8)()
    for n in range(8):
        strides[n] = _lib.NeoxStrides(4 * 128 * 192, 128 * 192, 192)
    a = make_args(strides=ctypes.cast(strides, ctypes.POINTER(_lib.NeoxStrides)))
    # valid strides: validation passes, so the call stops at the device check on a CPU host
    st = lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None)
    assert st in (OK, E_DEV)
    strides[1] = _lib.NeoxStrides(4 * 128 * 192, 128 * 192, 100)  # k rows not 16-byte aligned
    assert lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None) == E_ALIGN
    strides[1] = _lib.NeoxStrides(-1, 0, 64)
    assert lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None) == E_ARG


def test_null_args_struct(lib):
    assert lib.neox_attn_fwd_ex(None, A1, A2, A3, A4, A5, None, 0, None) == E_ARG
    assert lib.neox_attn_bwd_ex(None, A1, A2, A3, A4, A5, A6, A7, A8, A9, A1, 1 << 30,
                                None) == E_ARG


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present on this host")
def test_valid_call_without_gpu_fails_loudly(lib):
    """On a host without a GPU a fully valid call must return NEOX_E_DEVICE
    (never silently compute anything elsewhere)."""
    assert fwd(lib) == E_DEV
    assert bwd(lib) == E_DEV


def test_workspace_size_is_linear_in_sequence_length(lib):
    """O(n) memory: the backward workspace is the rotated q and k (2 bytes per
    element; the fp32 path's dq accumulator lies over the same bytes) and two
    fp32 row terms, each part rounded up to 256 bytes, with no S^2 term: the
    forward workspace plus 8 bytes per row."""
    def r256(n):
        return ((n + 255) // 256) * 256
    for (B, H, D) in [(1, 1, 64), (4, 64, 96), (1, 32, 128), (3, 5, 96)]:
        for S in (1, 17, 2048, 16384, 1 << 20):
            rows = B * H * S
            rot = 2 * r256(rows * D * 2)
            acc = r256(rows * D * 4)
            assert acc <= rot  # the fp32 accumulator fits over the rotated rows
            expect = rot + 2 * r256(rows * 4)
            assert lib.neox_rope_attn_bwd_workspace_size(B, H, S, D) == expect
            if rows * D < (1 << 31):
                fwd = lib.neox_rope_attn_fwd_workspace_size(B, H, S, D)
                assert fwd == rot and expect - fwd == 2 * r256(rows * 4)
    assert lib.neox_rope_attn_bwd_workspace_size(0, 1, 1, 64) == 0
    assert lib.neox_rope_attn_bwd_workspace_size(1 << 16, 1 << 8, 1 << 8, 64) == 0


def test_check_doc_offsets(lib):
    def chk(rows, S):
        arr = np.ascontiguousarray(rows, dtype=np.int32)
        return lib.neox_check_doc_offsets(arr.ctypes.data_as(P), arr.shape[0], arr.shape[1] - 1, S)
    assert chk([[0, 10, 10, 30]], 30) == OK
    assert chk([[0, 30], [0, 30]], 30) == OK
    assert chk([[1, 30]], 30) == E_ARG
    assert chk([[0, 29]], 30) == E_ARG
    assert chk([[0, 20, 10, 30]], 30) == E_ARG
    assert lib.neox_check_doc_offsets(None, 1, 1, 30) == E_ARG


def test_rope_table_prepare_validation(lib):
    assert lib.neox_rope_table_prepare(0, 16, 1e4) == E_ARG
    assert lib.neox_rope_table_prepare(128, 15, 1e4) == E_ARG
    assert lib.neox_rope_table_prepare(128, 16, -1.0) == E_ARG
    assert lib.neox_rope_table_prepare(128, -2, 1e4) == E_ARG
    assert lib.neox_rope_table_prepare(128, 16, float("nan")) == E_ARG
    assert lib.neox_rope_table_prepare(128, 0, 1e4) == OK  # nothing to build
    if not os.path.exists("/dev/kfd"):
        assert lib.neox_rope_table_prepare(128, 16, 1e4) == E_DEV


@pytest.mark.gpu
def test_unprepared_rotary_table_is_an_error_and_enqueues_nothing(lib):
    """Compute calls never allocate: a RoPE call whose (rotary_dim, rope_base,
    length) has no prepared table returns NEOX_E_NOT_PREPARED before touching
    any buffer; after neox_rope_table_prepare the same call runs.  A table
    prepared for a longer length serves shorter ones; rotary_dim = 0 and ALiBi
    need none."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_neox_amd as neox
    # a base no other test prepares; tables are built for whole multiples of 256
    # positions, so S // 2 = 150 gets a 256-position table, short of S = 300
    B, H, S, D, rd, base = 1, 2, 300, 64, 16, 4321.5
    q, k, v, do = (torch.randn(B, H, S, D, device="cuda").to(torch.bfloat16) for _ in range(4))
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, S), 7.0, device="cuda")
    ws = torch.zeros(neox.neox_rope_attn_bwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                     device="cuda")
    grads = [torch.full_like(q, 7.0) for _ in range(3)]
    dec_ws = torch.zeros(neox.neox_rope_attn_decode_workspace_size(B, H, D, S),
                         dtype=torch.uint8, device="cuda")
    lens = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    kc, vc = k.clone(), v.clone()
    o1 = torch.full((B, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((B, H), 7.0, device="cuda")

    def calls(length):
        qq, kk, vv, oo, ll, dd = (t[:, :, :length] for t in (q, k, v, o, lse, do))
        gg = [g[:, :, :length] for g in grads]
        with pytest.raises(neox.NeoxError) as e1:
            neox.neox_rope_attn_fwd(qq, kk, vv, oo, ll, rd, base, workspace=ws)
        with pytest.raises(neox.NeoxError) as e2:
            neox.neox_attn_fwd_ex(qq, kk, vv, oo, ll, rotary_dim=rd, rope_base=base)
        with pytest.raises(neox.NeoxError) as e3:
            neox.neox_rope_attn_bwd(qq, kk, vv, oo, dd, ll, *gg, rd, base, workspace=ws)
        with pytest.raises(neox.NeoxError) as e4:
            neox.neox_attn_bwd_ex(qq, kk, vv, oo, dd, ll, *gg, rotary_dim=rd, rope_base=base,
                                  workspace=ws)
        return [e.value.status for e in (e1, e2, e3, e4)]

    torch.cuda.synchronize()
    assert calls(S) == [E_NOT_PREPARED] * 4
    with pytest.raises(neox.NeoxError) as e5:
        neox.neox_rope_attn_decode(*(t[:, :, 0].contiguous() for t in (q, k, v)), kc, vc, lens,
                                   o1, l1, rd, base, workspace=dec_ws)
    assert e5.value.status == E_NOT_PREPARED
    neox.neox_rope_table_prepare(S // 2, rd, base)
    assert calls(S) == [E_NOT_PREPARED] * 4  # the table is shorter than S
    torch.cuda.synchronize()
    for t in [o, lse, o1, l1] + grads:
        assert bool((t == 7.0).all()), "a refused call wrote an output"
    assert bool((ws == 0).all()) and bool((dec_ws == 0).all())
    assert bool(torch.equal(kc, k)) and bool(torch.equal(vc, v))
    # a table for S covers every shorter length
    neox.neox_rope_table_prepare(S, rd, base)
    neox.neox_rope_table_prepare(S // 4, rd, base)  # already covered: no new table
    for length in (S, S // 2, 33):
        qq, kk, vv = (t[:, :, :length].contiguous() for t in (q, k, v))
        oo = torch.empty_like(qq)
        ll = torch.empty((B, H, length), device="cuda")
        neox.neox_attn_fwd_ex(qq, kk, vv, oo, ll, rotary_dim=rd, rope_base=base)
        torch.cuda.synchronize()
        assert bool(oo.isfinite().all()) and bool(ll.isfinite().all())
    q1, k1, v1 = (t[:, :, 0].contiguous() for t in (q, k, v))
    neox.neox_rope_attn_decode(q1, k1, v1, kc, vc, lens, o1, l1, rd, base, workspace=dec_ws)
    # no table needed without rotation or with ALiBi
    neox.neox_attn_fwd_ex(q, k, v, o, lse, rotary_dim=0, rope_base=base)
    neox.neox_attn_fwd_ex(q, k, v, o, lse, pos=neox.NEOX_POS_ALIBI)
    torch.cuda.synchronize()
    assert bool(o.isfinite().all()) and bool(o1.isfinite().all())


def test_generated_doc_layout_is_valid(lib):
    from causal_attention_neox_amd.workloads import WORKLOADS, generate
    wl = WORKLOADS["alibi_docs_s4096_d128"].with_sizes(H=1, D=64)
    inp = generate(wl, with_dout=False)
    offs = inp.doc_offsets
    arr = np.ascontiguousarray(offs)
    assert lib.neox_check_doc_offsets(arr.ctypes.data_as(P), arr.shape[0], arr.shape[1] - 1,
                                      wl.S) == OK
    for row in offs:
        lengths = np.diff(row)
        lengths = lengths[lengths > 0]
        assert lengths.sum() == wl.S
        assert lengths.min() >= wl.doc_min and lengths.max() <= wl.doc_max


def dec(lib, q=A1, k=A2, v=A3, kc=A4, vc=A5, lens=A6, o=A7, lse=A8, B=2, H=4, D=64, cap=300,
        rd=16, base=1e4, scale=0.125, dtype=BF16, ws=None, wsb=None):
    need = lib.neox_rope_attn_decode_workspace_size(B, H, D, cap)
    ws = P(0x100000) if ws is None else ws
    wsb = need if wsb is None else wsb
    return lib.neox_rope_attn_decode(q, k, v, kc, vc, lens, o, lse, B, H, D, cap, rd, base,
                                     scale, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_ARG), (dict(kc=None), E_ARG), (dict(lens=None), E_ARG),
    (dict(lse=None), E_ARG), (dict(B=0), E_ARG), (dict(cap=0), E_ARG), (dict(D=0), E_ARG),
    (dict(D=80), E_UNSUP), (dict(rd=15), E_ARG), (dict(rd=66), E_ARG),
    (dict(base=0.0), E_ARG), (dict(scale=float("inf")), E_ARG), (dict(dtype=3), E_ARG),
    (dict(o=A1), E_ARG), (dict(o=A4), E_ARG), (dict(vc=P(0x50008)), E_ALIGN),
    (dict(lens=P(0x60004)), E_ALIGN), (dict(ws=P(0)), E_WS), (dict(wsb=64), E_WS),
    (dict(ws=P(0x100010)), E_ALIGN), (dict(B=1 << 12, H=1 << 10, cap=1 << 10), E_ARG),
])
def test_decode_validation(lib, kw, status):
    assert dec(lib, **kw) == status


def test_decode_workspace_size(lib):
    """(m, l, o[D]) fp32 partials, 16-byte aligned records, one per 256-row
    chunk of the cache, rounded up to 256 bytes."""
    def r256(n):
        return ((n + 255) // 256) * 256
    for (B, H, D, cap) in [(1, 1, 64, 1), (2, 4, 96, 256), (16, 64, 96, 2048), (3, 5, 128, 257)]:
        nsplit = (cap + 255) // 256
        expect = r256(B * H * nsplit * (D + 4) * 4)
        assert lib.neox_rope_attn_decode_workspace_size(B, H, D, cap) == expect
    assert lib.neox_rope_attn_decode_workspace_size(0, 1, 64, 16) == 0
    assert lib.neox_rope_attn_decode_workspace_size(1, 1, 64, 0) == 0
    assert lib.neox_rope_attn_decode_workspace_size(1 << 12, 1 << 10, 64, 1 << 10) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present on this host")
def test_valid_decode_without_gpu_fails_loudly(lib):
    assert dec(lib) == E_DEV


def fp8(lib, q=A1, k=A2, v=A3, qs=0.01, ks=0.01, vs=0.01, o=A4, lse=A5, B=2, H=4, S=128, D=128,
        causal=1, scale=0.088, out=0):
    return lib.neox_attn_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, H, S, D, causal, scale, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_ARG), (dict(lse=None), E_ARG), (dict(B=0), E_ARG), (dict(S=0), E_ARG),
    (dict(D=80), E_UNSUP), (dict(qs=0.0), E_ARG), (dict(vs=float("nan")), E_ARG),
    (dict(ks=-1.0), E_ARG), (dict(scale=0.0), E_ARG), (dict(out=5), E_ARG),
    (dict(o=A1), E_ARG), (dict(v=P(0x30008)), E_ALIGN), (dict(lse=P(0x50004)), E_ALIGN),
    (dict(B=1 << 16, H=1 << 8, S=1 << 8), E_ARG),
])
def test_fp8_forward_validation(lib, kw, status):
    assert fp8(lib, **kw) == status


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present on this host")
def test_valid_fp8_forward_without_gpu_fails_loudly(lib):
    assert fp8(lib) == E_DEV


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more ends with a message and
    a non-zero status before any GPU work."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_noalloc_decode_validation(lib):
    """The no-allocation decode checks its arguments like the workspace one and
    refuses problems whose partials exceed its fixed array, before any device
    work (so on a host without a GPU only a fitting call reaches E_DEV)."""
    def call(B=2, H=4, D=64, cap=300, rd=16, q=A1, o=A7):
        return lib.neox_rope_attn_decode_noalloc(q, A2, A3, A4, A5, A6, o, A8, B, H, D, cap, rd,
                                                 1e4, 0.125, BF16, None)
    assert call(q=None) == E_ARG
    assert call(o=A1) == E_ARG
    assert call(D=80) == E_UNSUP
    big = (8, 64, 96, 16384)
    assert lib.neox_rope_attn_decode_workspace_size(*big) > _lib.NEOX_DECODE_SCRATCH_BYTES
    assert call(B=8, H=64, D=96, cap=16384) == -9
    fits = (8, 64, 96, 8192)
    assert lib.neox_rope_attn_decode_workspace_size(*fits) <= _lib.NEOX_DECODE_SCRATCH_BYTES
    if not os.path.exists("/dev/kfd"):
        assert call(B=8, H=64, D=96, cap=8192) == E_DEV
    assert lib.neox_status_str(-9) != b"unknown status"


def test_ex_row_stride_bound(lib):
    """Row strides beyond 2^22 elements are refused before any device work."""
    strides = (_lib.NeoxStrides * 8)()
    for n in range(8):
        strides[n] = _lib.NeoxStrides(4 * 128 * 192, 128 * 192, 192)
    strides[0] = _lib.NeoxStrides(0, 0, (1 << 22) + 8)
    a = make_args(strides=ctypes.cast(strides, ctypes.POINTER(_lib.NeoxStrides)))
    assert lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None) == E_UNSUP
    strides[0] = _lib.NeoxStrides(0, 0, 1 << 22)
    assert lib.neox_attn_fwd_ex(ctypes.byref(a), A1, A2, A3, A4, A5, None, 0, None) in (OK, E_DEV)


def plan(lib, **kw):
    ws = kw.pop("ws", 1)
    a = make_args(**kw)
    out = _lib.NeoxPlan()
    st = lib.neox_attn_plan(ctypes.byref(a), ws, ctypes.byref(out))
    return st, {n: getattr(out, n) for n, _ in _lib.NeoxPlan._fields_}


@pytest.mark.parametrize("kw,expect", [
    # with a forward workspace: the row pass, then the rotation-free kernel
    (dict(D=96, rotary_dim=24), dict(fwd_rotation_pass=1, fwd_k_staging=0, fwd_rotate_q=0)),
    (dict(D=128, rotary_dim=128), dict(fwd_rotation_pass=1, fwd_k_staging=0, fwd_rotate_q=0)),
    # without one: the kernel rotates Q~ and stages K by the rotary width
    (dict(D=128, rotary_dim=128, ws=0), dict(fwd_rotation_pass=0, fwd_k_staging=1, fwd_rotate_q=1)),
    (dict(D=64, rotary_dim=16, ws=0), dict(fwd_k_staging=1, fwd_rotate_q=1)),
    (dict(D=96, rotary_dim=24, ws=0), dict(fwd_k_staging=2, fwd_rotate_q=1)),
    (dict(D=128, rotary_dim=40, ws=0), dict(fwd_k_staging=2, fwd_rotate_q=1)),
    (dict(D=96, rotary_dim=6, ws=0), dict(fwd_k_staging=3, fwd_rotate_q=1)),
    (dict(D=64, rotary_dim=2, ws=0), dict(fwd_k_staging=3, fwd_rotate_q=1)),
    # no rotation, ALiBi, fp32
    (dict(rotary_dim=0), dict(fwd_rotation_pass=0, fwd_k_staging=0, fwd_rotate_q=0,
                              bwd_rotation_pass=0)),
    (dict(rotary_dim=0, ws=0), dict(fwd_rotation_pass=0, fwd_k_staging=0, fwd_rotate_q=0)),
    (dict(pos=2, rotary_dim=0), dict(alibi=1, fwd_rotation_pass=0, fwd_k_staging=0,
                                     bwd_rotation_pass=0)),
    (dict(dtype=F32, rotary_dim=16), dict(fp32_path=1, fwd_rotation_pass=0, fwd_rotate_q=0)),
    (dict(dtype=2, rotary_dim=24, D=96, ws=0), dict(fp32_path=0, fwd_k_staging=2)),
    # backward: rotates q, k itself unless the forward's rotated rows are reused
    (dict(rotary_dim=16), dict(bwd_rotation_pass=1)),
    (dict(rotary_dim=16, reuse_rotated_qk=1), dict(bwd_rotation_pass=0)),
])
def test_kernel_plan(lib, kw, expect):
    """The host-side choice of kernel forms (shared by the launchers)."""
    st, got = plan(lib, **kw)
    assert st == OK
    for k, v in expect.items():
        assert got[k] == v, (k, got)


def test_kernel_plan_validation(lib):
    assert plan(lib, D=80)[0] == E_UNSUP
    assert plan(lib, rotary_dim=15)[0] == E_ARG
    assert plan(lib, ws=2)[0] == E_ARG
    assert lib.neox_attn_plan(None, 1, None) == E_ARG
    a = make_args()
    assert lib.neox_attn_plan(ctypes.byref(a), 1, None) == E_ARG
