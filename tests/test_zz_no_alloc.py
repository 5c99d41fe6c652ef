"""The no-allocation decode entry point against the workspace one.

neox_rope_attn_decode_noalloc runs the same kernels with its chunk partials
in the library's fixed per-device array, so its outputs and the cache rows it
writes must equal those of neox_rope_attn_decode bit for bit.  Two calls in a
row, the second smaller than the first, both split over several chunks (so
the array is used, and the second call runs over what the first left there);
then a problem past the array's size is refused before any work.
"""

import numpy as np
import pytest

from causal_attention_neox_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_neox_amd._lib as L
    L.load()
    return torch


def _dev(torch, arr, dtype):
    if dtype in (W.BF16, W.F16):
        tdt = torch.bfloat16 if dtype == W.BF16 else torch.float16
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(tdt).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _same(torch, a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _both(torch, neox, wl):
    """Runs both entry points on identical inputs and caches; returns the
    (workspace, no-allocation) results."""
    inp = W.generate_decode(wl)
    dt = wl.dtype
    q, k, v = (_dev(torch, getattr(inp, n), dt) for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp.lens.copy()).cuda()
    neox.neox_rope_table_prepare(wl.cap, wl.rotary_dim, wl.rope_base)
    out = []
    for noalloc in (False, True):
        kc, vc = _dev(torch, inp.k_cache, dt), _dev(torch, inp.v_cache, dt)
        o = torch.full((wl.B, wl.H, wl.D), float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((wl.B, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            neox.neox_rope_attn_decode_noalloc(q, k, v, kc, vc, lens, o, lse, wl.rotary_dim,
                                               wl.rope_base, wl.softmax_scale)
        else:
            ws = torch.empty(neox.neox_rope_attn_decode_workspace_size(wl.B, wl.H, wl.D, wl.cap),
                             dtype=torch.uint8, device="cuda")
            neox.neox_rope_attn_decode(q, k, v, kc, vc, lens, o, lse, wl.rotary_dim,
                                       wl.rope_base, wl.softmax_scale, workspace=ws)
        torch.cuda.synchronize()
        out.append((o, lse, kc, vc))
    return out


def test_noalloc_decode_equals_workspace_decode_on_consecutive_calls(torch):
    import causal_attention_neox_amd as neox
    cases = [
        # first call: 16 heads, 4096-row cache -> 16 chunks of 256 rows each head
        W.DecodeWorkload("noalloc_a", B=2, H=8, D=128, rotary_dim=32, cap=4096, dtype=W.BF16,
                         lens="ragged", seed=901),
        # second call, smaller: 4 heads, 1000-row cache -> 4 chunks
        W.DecodeWorkload("noalloc_b", B=1, H=4, D=96, rotary_dim=24, cap=1000, dtype=W.BF16,
                         lens="ragged", seed=902),
    ]
    for wl in cases:
        print(f"[noalloc] {wl.name} B={wl.B} H={wl.H} D={wl.D} cap={wl.cap}", flush=True)
        assert neox.neox_rope_attn_decode_workspace_size(wl.B, wl.H, wl.D, wl.cap) <= \
            neox._lib.NEOX_DECODE_SCRATCH_BYTES
        (o0, l0, k0, v0), (o1, l1, k1, v1) = _both(torch, neox, wl)
        assert bool(o0.isfinite().all()) and bool(l0.isfinite().all())
        assert _same(torch, o1, o0), f"{wl.name}: o differs"
        assert _same(torch, l1, l0), f"{wl.name}: lse differs"
        assert _same(torch, k1, k0) and _same(torch, v1, v0), f"{wl.name}: caches differ"


def test_noalloc_decode_refuses_problems_beyond_its_array(torch):
    import causal_attention_neox_amd as neox
    B, H, D, cap = 8, 64, 96, 16384  # 12.5 MiB of partials > 8 MiB
    assert neox.neox_rope_attn_decode_workspace_size(B, H, D, cap) > \
        neox._lib.NEOX_DECODE_SCRATCH_BYTES
    small = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((B, H, 1, D), dtype=torch.bfloat16, device="cuda").expand(B, H, cap, D)
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    o = torch.empty_like(small)
    lse = torch.empty((B, H), device="cuda")
    with pytest.raises(neox.NeoxError) as e:
        neox.neox_rope_attn_decode_noalloc(small, small, small, cache, cache, lens, o, lse, 0)
    assert e.value.status == neox._lib.NEOX_E_TOO_LARGE
