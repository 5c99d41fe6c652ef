"""Helpers shared by the GPU parity tests: run the library on generated inputs
and compare against the CPU oracle."""

from __future__ import annotations

import concurrent.futures
import multiprocessing
import os

import numpy as np

import causal_attention_neox_amd as neox
from causal_attention_neox_amd.workloads import BF16, F16, F32, Inputs, Workload, storage_to_f64
from oracle import neox_oracle as orc

# Accuracy bars: fp32 storage max-abs 1e-5; bf16 storage max-abs 2e-2 and
# mean-abs 2e-3, on o, dq, dk and dv.  fp16 storage: the bf16 bars scaled by the
# ratio of the unit roundoffs (2^-11 / 2^-8 = 1/8): max-abs 2.5e-3, mean-abs
# 2.5e-4.  lse is held to the same max-abs bar.
TOL = {"f32": dict(max_abs=1e-5, mean_abs=1e-5), "bf16": dict(max_abs=2e-2, mean_abs=2e-3),
       "f16": dict(max_abs=2.5e-3, mean_abs=2.5e-4)}


def torch_mod():
    import torch
    return torch


def to_device(inp: Inputs, name: str):
    torch = torch_mod()
    arr = getattr(inp, name)
    if inp.wl.dtype in (BF16, F16):
        tdt = torch.bfloat16 if inp.wl.dtype == BF16 else torch.float16
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(tdt).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_library(inp: Inputs, backward: bool = True, out_f32: bool = False, force_ex: bool = False,
                fwd_workspace: bool = True, reuse_qk: bool = False):
    """Forward (and backward) on the GPU through the C ABI; returns torch tensors.
    ``fwd_workspace`` gives the forward its optional workspace (pre-rotated queries and keys);
    ``reuse_qk`` runs the forward in the backward's workspace and lets the backward
    reuse the rotated rows it leaves there."""
    torch = torch_mod()
    wl = inp.wl
    q, k, v = (to_device(inp, n) for n in ("q", "k", "v"))
    odt = torch.float32 if (out_f32 or wl.dtype == F32) else q.dtype
    o = torch.empty(q.shape, dtype=odt, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    docs = None if inp.doc_offsets is None else torch.from_numpy(inp.doc_offsets).cuda()
    use_ex = force_ex or wl.alibi or docs is not None or out_f32
    pos = neox.NEOX_POS_ALIBI if wl.alibi else neox.NEOX_POS_ROPE
    kw = dict(pos=pos, rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
              softmax_scale=wl.softmax_scale, doc_offsets=docs, out_f32=out_f32)
    B, H, S, D = q.shape
    if not wl.alibi:
        neox.neox_rope_table_prepare(S, wl.rotary_dim, wl.rope_base)
    fws = None
    ws = torch.empty(neox.neox_rope_attn_bwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                     device="cuda")
    if reuse_qk:
        use_ex = True
        fws = ws
    elif fwd_workspace:
        fws = torch.empty(neox.neox_rope_attn_fwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                          device="cuda")
    if use_ex:
        neox.neox_attn_fwd_ex(q, k, v, o, lse, workspace=fws, **kw)
    else:
        neox.neox_rope_attn_fwd(q, k, v, o, lse, wl.rotary_dim, wl.rope_base, wl.causal,
                                wl.softmax_scale, workspace=fws)
    res = {"o": o, "lse": lse}
    if backward:
        do = to_device(inp, "dout")
        o_in = o if o.dtype == q.dtype else o.to(q.dtype)
        dq, dk, dv = (torch.empty(q.shape, dtype=odt, device="cuda") for _ in range(3))
        if use_ex:
            neox.neox_attn_bwd_ex(q, k, v, o_in, do, lse, dq, dk, dv, workspace=ws,
                                  reuse_rotated_qk=reuse_qk, **kw)
        else:
            neox.neox_rope_attn_bwd(q, k, v, o_in, do, lse, dq, dk, dv, wl.rotary_dim,
                                    wl.rope_base, wl.causal, wl.softmax_scale, workspace=ws)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def oracle_heads(inp: Inputs, heads, backward: bool = True):
    """Oracle outputs for the listed (b, h) heads: dict of [n, S, D] / [n, S]."""
    wl = inp.wl
    sel = lambda name: np.stack([_widen(inp, name, b, h) for b, h in heads])[:, None]  # noqa: E731
    q, k, v = sel("q"), sel("k"), sel("v")
    out = {}
    slopes_all = orc.alibi_slopes(wl.H) if wl.alibi else None
    res = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    for n, (b, h) in enumerate(heads):
        kw = dict(rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
                  softmax_scale=wl.softmax_scale, rope_doc_positions=wl.rope_doc_positions,
                  alibi=False if slopes_all is None else slopes_all[h:h + 1],
                  doc_offsets=None if inp.doc_offsets is None else inp.doc_offsets[b:b + 1])
        if backward:
            do = _widen(inp, "dout", b, h)[None, None]
            o, lse, dq, dk, dv = orc.attn_bwd(q[n:n + 1], k[n:n + 1], v[n:n + 1], do, **kw)
            for key, val in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv)):
                res[key].append(val[0, 0])
        else:
            o, lse = orc.attn_fwd(q[n:n + 1], k[n:n + 1], v[n:n + 1], **kw)
            res["o"].append(o[0, 0])
            res["lse"].append(lse[0, 0])
    for key, val in res.items():
        if val:
            out[key] = np.stack(val)
    return out


def _widen(inp: Inputs, name: str, b: int, h: int) -> np.ndarray:
    return storage_to_f64(getattr(inp, name)[b, h], inp.wl.dtype)


def compare(gpu: dict, ref: dict, heads, dtype: str, names=None, label: str = ""):
    """Max-abs / mean-abs per output against the bars; returns the stats."""
    tol = TOL[dtype]
    stats = {}
    failures = []
    for name in names or ref.keys():
        g = to_f64(gpu[name])
        g = np.stack([g[b, h] for b, h in heads])
        r = ref[name]
        assert g.shape == r.shape, (name, g.shape, r.shape)
        if not np.all(np.isfinite(g)):
            failures.append(f"{name}: non-finite values")
            continue
        err = np.abs(g - r)
        mx, mean = float(err.max()), float(err.mean())
        stats[name] = (mx, mean, float(np.abs(r).max()))
        if mx > tol["max_abs"] or (name != "lse" and mean > tol["mean_abs"]):
            idx = np.unravel_index(int(err.argmax()), err.shape)
            failures.append(f"{name}: max_abs {mx:.3e} mean_abs {mean:.3e} at {idx} "
                            f"(gpu {g[idx]:.6f} ref {r[idx]:.6f})")
    line = " ".join(f"{k}=({v[0]:.2e},{v[1]:.2e},|ref|max {v[2]:.2f})" for k, v in stats.items())
    print(f"[parity] {label} {line}", flush=True)
    assert not failures, f"{label}: " + "; ".join(failures)
    return stats


def small_workload(B, H, S, D, rd, dtype="bf16", causal=True, alibi=False, docs=None, seed=7,
                   amp=1.0) -> Workload:
    return Workload(f"case_b{B}h{H}s{S}d{D}rd{rd}", B=B, H=H, S=S, D=D, rotary_dim=rd,
                    dtype=dtype, causal=causal, alibi=alibi, packed_docs=docs is not None,
                    doc_min=docs[0] if docs else 64, doc_max=docs[1] if docs else 4096, seed=seed,
                    amp=amp)


# ---------------------------------------------------------------- many heads

def _oracle_one_head(args):
    """One head through the oracle in a worker process (float64 inputs)."""
    q, k, v, do, kw, backward = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):  # one core per worker process
        if backward:
            return tuple(x[0, 0] for x in orc.attn_bwd(q, k, v, do, **kw))
        return tuple(x[0, 0] for x in orc.attn_fwd(q, k, v, **kw))


def _head_args(inp: Inputs, b: int, h: int, backward: bool):
    wl = inp.wl
    slopes = orc.alibi_slopes(wl.H) if wl.alibi else None
    kw = dict(rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
              softmax_scale=wl.softmax_scale, rope_doc_positions=wl.rope_doc_positions,
              alibi=False if slopes is None else slopes[h:h + 1],
              doc_offsets=None if inp.doc_offsets is None else inp.doc_offsets[b:b + 1])
    sel = lambda name: _widen(inp, name, b, h)[None, None]  # noqa: E731
    return (sel("q"), sel("k"), sel("v"), sel("dout") if backward else None, kw, backward)


def oracle_workers(S: int) -> int:
    """Worker processes for the oracle: the host's cores, at most 16 (the share
    of one GPU on the test machines), fewer for long sequences (each head holds
    several S x S float64 matrices)."""
    n = min(16, os.cpu_count() or 1)
    if S > 8192:
        n = min(n, 4)
    return max(1, n)


def compare_many_heads(gpu: dict, inp: Inputs, heads, dtype: str, label: str = "",
                       backward: bool = True, out_f32_bars: bool = False):
    """Every listed head of the GPU outputs against the oracle, computed in
    parallel worker processes (spawned: the GPU context is not inherited) and
    compared as each head arrives; returns the stats dict of compare().
    The bars are those of `dtype`."""
    names = ("o", "lse", "dq", "dk", "dv") if backward else ("o", "lse")
    g = {n: to_f64(gpu[n]) for n in names}  # one host copy of every output
    tol = TOL[dtype]
    mx = {n: 0.0 for n in names}
    sm = {n: 0.0 for n in names}
    cnt = {n: 0 for n in names}
    refmax = {n: 0.0 for n in names}
    worst = {}
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=oracle_workers(inp.wl.S),
                                                mp_context=ctx) as ex:
        futs = {ex.submit(_oracle_one_head, _head_args(inp, b, h, backward)): (b, h)
                for b, h in heads}
        for fut in concurrent.futures.as_completed(futs):
            b, h = futs[fut]
            ref = fut.result()
            for n, r in zip(names, ref):
                x = g[n][b, h]
                assert np.all(np.isfinite(x)), f"{label}: non-finite {n} at head {(b, h)}"
                err = np.abs(x - r)
                m = float(err.max())
                if m > mx[n]:
                    mx[n] = m
                    worst[n] = (b, h) + tuple(int(i) for i in np.unravel_index(int(err.argmax()), err.shape))
                sm[n] += float(err.sum())
                cnt[n] += err.size
                refmax[n] = max(refmax[n], float(np.abs(r).max()))
    stats = {n: (mx[n], sm[n] / cnt[n], refmax[n]) for n in names}
    line = " ".join(f"{k}=({v[0]:.2e},{v[1]:.2e},|ref|max {v[2]:.2f})" for k, v in stats.items())
    print(f"[parity] {label} ({len(heads)} heads) {line}", flush=True)
    failures = [f"{n}: max_abs {stats[n][0]:.3e} mean_abs {stats[n][1]:.3e} worst at {worst.get(n)}"
                for n in names
                if stats[n][0] > tol["max_abs"] or (n != "lse" and stats[n][1] > tol["mean_abs"])]
    assert not failures, f"{label}: " + "; ".join(failures)
    return stats


def spread_heads(B: int, H: int, n: int):
    """n heads (b, h) spread over the B*H heads so that every residue of the
    flat head index modulo 8 (the XCD a head's workgroups run on) appears, and
    the first and last heads are included."""
    BH = B * H
    if n >= BH:
        return [(i // H, i % H) for i in range(BH)]
    idx = sorted(set([0, BH - 1] + [int(round(j * (BH - 1) / (n - 1))) for j in range(n)] +
                     [x for x in range(8) if x < BH]))
    return [(i // H, i % H) for i in idx]
