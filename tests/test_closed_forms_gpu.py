"""Full-size GPU checks against closed forms, on every head (no oracle run).

The method is exact attention ("GPT-NeoX 开源训练框架深度解读", section
"问题二：注意力计算太慢": FlashAttention keeps the mathematical result), so
inputs chosen to make the softmax trivial have results that follow from the
definition in O(S D) per head:

* q = 0: every allowed score is the bias alone, so o_i is the mean of the
  values v_j over the allowed keys of row i (with ALiBi the mean weighted by
  e^(-m (i - j))) and lse_i = ln(number of allowed keys) (with ALiBi the log of
  the sum of those weights);
* v_j = c for every key (c constant along the sequence): o_i = c, and since
  dP_ij = dO_i . c does not depend on j, dS = P (dP - Delta) = 0, so dq = dk = 0;
* any inputs: the rows of P sum to one, so sum_j dv_j = sum_i dO_i within
  every document, and the first row of a document attends to itself alone,
  so its o equals its v bit for bit.

Also the canary check: every output written through views into larger
buffers whose bands before and after are filled with a pattern; the bands
must come back unchanged.
"""

import numpy as np
import pytest

from causal_attention_neox_amd.workloads import WORKLOADS, generate, storage_to_f64
from oracle import neox_oracle as orc
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

CLOSED = ["neox20b_s2048_h64_d96_rd24", "long_s16384_d128", "alibi_docs_s4096_d128"]

@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_neox_amd._lib as L
    L.load()
    return torch

def _doc_starts(inp, b):
    """Start of the document holding each position of batch row b."""
    S = inp.wl.S
    if inp.doc_offsets is None:
        return np.zeros(S, dtype=np.int64)
    off = inp.doc_offsets[b].astype(np.int64)
    idx = np.searchsorted(off, np.arange(S), side="right") - 1
    return off[idx]

def _prefix_forms(inp, v64):
    """Closed forms for q = 0: o [B,H,S,D] and lse [B,H,S] (float64)."""
    wl = inp.wl
    B, H, S, D = v64.shape
    o = np.empty_like(v64)
    lse = np.empty((B, H, S))
    pos = np.arange(S)
    for b in range(B):
        start = _doc_starts(inp, b)
        first = pos == start
        if not wl.alibi:
            cnt = (pos - start + 1).astype(np.float64)
            cs = np.cumsum(v64[b], axis=1)  # [H, S, D]
            base = np.where(start > 0, start - 1, 0)
            before = np.where((start > 0)[None, :, None], cs[:, base, :], 0.0)
            o[b] = (cs - before) / cnt[None, :, None]
            lse[b] = np.log(cnt)[None, :]
        else:
            decay = np.exp(-orc.alibi_slopes(H))[:, None]  # [H, 1]
            acc = np.zeros((H, D))
            w = np.zeros(H)
            for i in range(S):
                if first[i]:
                    acc[:] = 0.0
                    w[:] = 0.0
                acc = acc * decay + v64[b, :, i, :]
                w = w * decay[:, 0] + 1.0
                o[b, :, i, :] = acc / w[:, None]
                lse[b, :, i] = np.log(w)
    return o, lse

def _stats(got, ref):
    err = np.abs(got - ref)
    return float(err.max()), float(err.mean())

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CLOSED)
def test_zero_queries_give_prefix_means(gpu, name):
    """q = 0 on every head: o is the (ALiBi-weighted) prefix mean of v within
    each document, lse its closed form."""
    wl = WORKLOADS[name]
    inp = generate(wl)
    inp.q = np.zeros_like(inp.q)
    res = pu.run_library(inp, backward=False)
    v64 = storage_to_f64(inp.v, wl.dtype)
    o_ref, lse_ref = _prefix_forms(inp, v64)
    mo, ao = _stats(pu.to_f64(res["o"]), o_ref)
    ml, al = _stats(pu.to_f64(res["lse"]), lse_ref)
    print(f"[closed] {name} q=0: o max {mo:.2e} mean {ao:.2e}; lse max {ml:.2e}", flush=True)
    assert mo <= 2e-2 and ao <= 2e-3, (mo, ao)
    assert ml <= 2e-2, ml

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CLOSED)
def test_constant_values_give_zero_query_and_key_gradients(gpu, name):
    """v constant along the sequence on every head: o = v, dq = dk = 0."""
    wl = WORKLOADS[name]
    inp = generate(wl)
    row = inp.v[:, :, :1, :]  # each head's first value row, repeated along S
    inp.v = np.ascontiguousarray(np.broadcast_to(row, inp.v.shape))
    res = pu.run_library(inp, backward=True, reuse_qk=True)
    c = storage_to_f64(inp.v, wl.dtype)
    mo, ao = _stats(pu.to_f64(res["o"]), c)
    mq, aq = _stats(pu.to_f64(res["dq"]), 0.0)
    mk, ak = _stats(pu.to_f64(res["dk"]), 0.0)
    print(f"[closed] {name} v=c: o max {mo:.2e}; dq max {mq:.2e} mean {aq:.2e}; "
          f"dk max {mk:.2e} mean {ak:.2e}", flush=True)
    assert mo <= 2e-2 and ao <= 2e-3
    assert mq <= 2e-2 and aq <= 2e-3
    assert mk <= 2e-2 and ak <= 2e-3

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CLOSED)
def test_value_gradient_sums_and_first_rows(gpu, name):
    """Regular inputs, every head: sum_j dv_j = sum_i dO_i in every document
    (within the rounding of the bf16 dv entries), and each document's first
    row has o = v exactly."""
    wl = WORKLOADS[name]
    inp = generate(wl)
    res = pu.run_library(inp, backward=True, reuse_qk=True)
    dv = pu.to_f64(res["dv"])
    o = pu.to_f64(res["o"])
    do = storage_to_f64(inp.dout, wl.dtype)
    v = storage_to_f64(inp.v, wl.dtype)
    worst = 0.0
    for b in range(wl.B):
        off = ([0, wl.S] if inp.doc_offsets is None
               else sorted(set(int(x) for x in inp.doc_offsets[b])))
        for s0, s1 in zip(off[:-1], off[1:]):
            if s1 <= s0:
                continue
            lhs = dv[b, :, s0:s1].sum(axis=1)
            rhs = do[b, :, s0:s1].sum(axis=1)
            # each stored dv entry carries at most half a bf16 spacing (2^-9
            # relative) and the kernel's fp32 error; 2^-7 sum |dv| bounds both
            bound = 2.0 ** -7 * np.abs(dv[b, :, s0:s1]).sum(axis=1) + 1e-2
            excess = np.abs(lhs - rhs) - bound
            worst = max(worst, float((np.abs(lhs - rhs) / bound).max()))
            assert np.all(excess <= 0), f"row {b} doc [{s0},{s1}): {float(excess.max()):.3e}"
            assert np.array_equal(o[b, :, s0], v[b, :, s0]), f"first row of doc {s0} in row {b}"
    print(f"[closed] {name}: sum dv vs sum dO worst at {worst:.3f} of its bound", flush=True)

@pytest.mark.parametrize("case", [(2, 3, 333, 96, 24, False), (1, 4, 300, 128, 0, True),
                                  (2, 2, 190, 64, 16, False)],
                         ids=["d96-rope", "d128-alibi", "d64-rope"])
def test_outputs_leave_canary_bands_untouched(gpu, case):
    """Outputs written through views into larger buffers: the 4 KiB bands
    before and after each output (and after the workspace) keep their fill."""
    torch = gpu
    import causal_attention_neox_amd as neox
    B, H, S, D, rd, alibi = case
    wl = pu.small_workload(B, H, S, D, 0 if alibi else rd, alibi=alibi, seed=S + 3)
    inp = generate(wl)
    q, k, v, do = (pu.to_device(inp, n) for n in ("q", "k", "v", "dout"))
    fill16 = -12345  # int16 pattern

    def guarded(shape, dtype, fill):
        n = int(np.prod(shape))
        per = 4 if dtype == torch.float32 else 2
        pad = 4096 // per
        buf = torch.full((pad + n + pad,), 0, dtype=dtype, device="cuda")
        buf.view(torch.int16 if per == 2 else torch.int32).fill_(fill)
        return buf, buf[pad:pad + n].view(shape), pad

    o_buf, o, po = guarded(q.shape, q.dtype, fill16)
    l_buf, lse, pl = guarded(q.shape[:3], torch.float32, -123456789)
    grads = [guarded(q.shape, q.dtype, fill16) for _ in range(3)]
    wsz = neox.neox_rope_attn_bwd_workspace_size(B, H, S, D)
    ws_buf = torch.full((wsz + 4096,), 77, dtype=torch.uint8, device="cuda")
    ws = ws_buf[:wsz]
    pos = neox.NEOX_POS_ALIBI if alibi else neox.NEOX_POS_ROPE
    kw = dict(pos=pos, rotary_dim=0 if alibi else rd)
    neox.neox_rope_table_prepare(S, kw["rotary_dim"])
    neox.neox_attn_fwd_ex(q, k, v, o, lse, workspace=ws, **kw)
    neox.neox_attn_bwd_ex(q, k, v, o, do, lse, grads[0][1], grads[1][1], grads[2][1],
                          workspace=ws, reuse_rotated_qk=not alibi, **kw)
    torch.cuda.synchronize()
    for buf, view, pad in [(o_buf, o, po), (l_buf, lse, pl)] + grads:
        raw = buf.view(torch.int16) if buf.dtype != torch.float32 else buf.view(torch.int32)
        fill = -123456789 if buf.dtype == torch.float32 else fill16
        n = view.numel()
        assert bool((raw[:pad] == fill).all()), "band before an output was written"
        assert bool((raw[pad + n:] == fill).all()), "band after an output was written"
        assert bool(torch.isfinite(view).all())
    assert bool((ws_buf[wsz:] == 77).all()), "band after the workspace was written"
