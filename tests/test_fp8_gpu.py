"""GPU parity of the FP8 (E4M3) forward (neox_attn_fwd_fp8) against the oracle.

The exact result is attention over the dequantised inputs (code x scale).  The
kernel rounds the probabilities to E4M3 before the P V product, a relative
error of at most 2^-4 per weight, so each output element may differ from the
exact one by up to 2^-4 sum_j p_ij |v_jd|: that sum is the oracle's attention
with |v| as values.  The bar per element adds the output rounding (bf16: 2^-8
relative, generous) and 1e-3 for probabilities below E4M3's normal range and
the matrix cores' fp32 accumulation.  lse is computed from fp32 scores of exact
FP8 products: held to 1e-3.
"""

import numpy as np
import pytest

from causal_attention_neox_amd import workloads as W
from oracle import neox_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_neox_amd._lib as L
    L.load()  # fails loudly when the library is missing
    return torch


def _run(torch, inp, out_f32=False):
    import causal_attention_neox_amd as neox
    wl = inp.wl
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (inp.q8, inp.k8, inp.v8))
    odt = torch.float32 if out_f32 else torch.bfloat16
    o = torch.empty((wl.B, wl.H, wl.S, wl.D), dtype=odt, device="cuda")
    lse = torch.empty((wl.B, wl.H, wl.S), dtype=torch.float32, device="cuda")
    neox.neox_attn_fwd_fp8(q8, k8, v8, *inp.scales, o, lse, causal=wl.causal,
                           softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, inp, heads, label, out_f32=False):
    wl = inp.wl
    sel = lambda a: np.stack([a[b, h] for b, h in heads])[:, None]  # noqa: E731
    q8, k8, v8 = sel(inp.q8), sel(inp.k8), sel(inp.v8)
    qs, ks, vs = inp.scales
    ref_o, ref_lse = orc.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, causal=wl.causal,
                                      softmax_scale=wl.softmax_scale)
    vabs = np.abs(orc.e4m3_decode(v8) * vs)
    o_abs, _ = orc.attn_fwd(orc.e4m3_decode(q8) * qs, orc.e4m3_decode(k8) * ks, vabs,
                            rotary_dim=0, causal=wl.causal, softmax_scale=wl.softmax_scale)
    g_o = np.stack([o[b, h] for b, h in heads])[:, None]
    g_lse = np.stack([lse[b, h] for b, h in heads])[:, None]
    assert np.all(np.isfinite(g_o)) and np.all(np.isfinite(g_lse)), f"{label}: non-finite"
    err = np.abs(g_o - ref_o)
    bound = 2.0 ** -4 * o_abs + (0.0 if out_f32 else 2.0 ** -8) * np.abs(ref_o) + 1e-3
    lerr = float(np.abs(g_lse - ref_lse).max())
    print(f"[fp8] {label} o max_abs {err.max():.3e} mean_abs {err.mean():.3e} "
          f"max err/bound {float((err / bound).max()):.3f} lse max_abs {lerr:.2e}", flush=True)
    idx = np.unravel_index(int((err / bound).argmax()), err.shape)
    assert np.all(err <= bound), f"{label}: o error {err[idx]:.3e} > bound {bound[idx]:.3e} at {idx}"
    assert lerr <= 1e-3, f"{label}: lse max_abs {lerr:.3e}"


SMALL = [
    # B, H, S, D, causal
    (1, 2, 1, 64, True),
    (1, 2, 65, 96, True),
    (2, 2, 130, 128, True),
    (1, 3, 257, 64, True),
    (1, 2, 190, 128, False),
    (1, 2, 300, 96, False),
    (1, 1, 129, 128, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'' if c[4] else '-noncausal'}"
                                              for c in SMALL])
def test_fp8_small_shapes_every_element(torch, case):
    B, H, S, D, causal = case
    inp = W.generate_fp8(W.Fp8Workload("case", B=B, H=H, S=S, D=D, causal=causal, seed=S + D))
    print(f"[fp8] case {case}", flush=True)
    o, lse = _run(torch, inp)
    heads = [(b, h) for b in range(B) for h in range(H)]
    _check(o, lse, inp, heads, f"{case}")


def test_fp8_fp32_output(torch):
    inp = W.generate_fp8(W.Fp8Workload("case", B=1, H=2, S=200, D=96, seed=9))
    o, lse = _run(torch, inp, out_f32=True)
    _check(o, lse, inp, [(0, 0), (0, 1)], "fp32 out", out_f32=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", sorted(W.FP8_WORKLOADS))
def test_fp8_full_size_sampled_heads(torch, name):
    inp = W.generate_fp8(W.FP8_WORKLOADS[name])
    print(f"[fp8] {name}: generated", flush=True)
    o, lse = _run(torch, inp)
    assert np.all(np.isfinite(o)), f"{name}: non-finite o"
    wl = inp.wl
    _check(o, lse, inp, [(0, 0), (wl.B - 1, wl.H - 1)], name)


def test_fp8_is_deterministic(torch):
    inp = W.generate_fp8(W.Fp8Workload("det", B=2, H=2, S=333, D=128, seed=4))
    a = _run(torch, inp)
    b = _run(torch, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
