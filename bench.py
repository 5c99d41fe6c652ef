#!/usr/bin/env python3
"""Benchmark of causal NeoX-rotary attention, forward + backward, on one MI355X.

One step = one forward and one backward call of the library over one batch of
the benchmark workload (the 2048-token context with the GPT-NeoX-20B head
layout: B=4, H=64, S=2048, D=96, 24 rotary dims, bf16), inputs resident in HBM.
W untimed warm-up steps, then K steps timed back to back with HIP events on the
launch stream, bracketed by device synchronisation.

value = algorithmic fwd+bwd FLOP per step / time per step, in TFLOP/s:
  4*D flop per allowed (query, key) pair for the forward (QK^T and PV) and
  10*D for the backward (QK^T and dO V^T recomputed, dV, dK, dQ); masked and
  skipped pairs, rotary and softmax arithmetic are not counted.

The JSON line also carries the roofline of the dominant kernel (timed live via
per-phase HIP events recorded by the library on the launch stream), the forward
efficiency at S=2048, D=128, the same step with fp16 storage, the FP8 forward at
S=2048, D=128, the decoding step's HBM rate (one new token per
sequence against a 2048-row cache), and the CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal RoPE-attention fwd+bwd TFLOP/s at S=2048 (1 GPU) + % of bf16 MFMA peak"
# Dense bf16 (and fp16) MFMA peak of MI355X: 256 CUs x 4096 flop/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
# Dense FP8 MFMA peak: twice the bf16 rate.
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the 20B layout)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-fwd-target", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with kernels of known traffic (scale for traffic counters)")
    return ap.parse_args()


def dev_tensor(torch, np, arr, dtype):
    if dtype in ("bf16", "f16"):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(tdt).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def make_events(torch, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # creates the underlying hipEvent_t
    return evs


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from profiles/traffic.json
    (FETCH_SIZE and WRITE_SIZE counters scaled by a plain copy), or None when
    absent or when the kernel's sources changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            ent = json.load(f)["kernels"][kernel]
        if ent["workload"] != workload or source_digest(ent["sources"]) != ent["sources_sha256"]:
            return None
        return int(ent["fetch_bytes"] + ent["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def run_gpu(args, torch, np, neox, W, wl, inp):
    q, k, v, do = (dev_tensor(torch, np, getattr(inp, n), wl.dtype) for n in ("q", "k", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, S, D = q.shape
    # One workspace for both calls: the forward leaves the rotated q and k in it
    # and the backward reuses them.
    ws = torch.empty(neox.neox_rope_attn_bwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                     device="cuda")
    docs = None if inp.doc_offsets is None else torch.from_numpy(inp.doc_offsets).cuda()
    pos = neox.NEOX_POS_ALIBI if wl.alibi else neox.NEOX_POS_ROPE
    kw = dict(pos=pos, rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
              softmax_scale=wl.softmax_scale, doc_offsets=docs)
    neox.neox_rope_table_prepare(S, kw["rotary_dim"], wl.rope_base)

    def step(ev):
        neox.neox_attn_fwd_ex(q, k, v, o, lse, workspace=ws, phase_events=ev[0:3], **kw)
        neox.neox_attn_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, workspace=ws,
                              phase_events=ev[3:7], reuse_rotated_qk=True, **kw)

    warm_ev = make_events(torch, 7)
    for _ in range(args.warmup):
        step(warm_ev)
    events = [make_events(torch, 7) for _ in range(args.steps)]
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(events[s])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    def avg(i, j):
        return sum(ev[i].elapsed_time(ev[j]) for ev in events) / len(events)

    # backward events: start, after the rotation pass (none here: q~ and k~ are
    # reused from the forward), after the dQ kernel (it also forms Delta and
    # the lse term), after the dK/dV kernel
    kernels_ms = {"fwd_rope_qk": avg(0, 1), "fwd": avg(1, 2), "bwd_dq": avg(4, 5),
                  "bwd_dkdv": avg(5, 6)}
    return total_ms, kernels_ms


def fwd_target(args, torch, np, neox, W):
    """Causal forward alone at S=2048, D=128 (full rotary), timed back to back."""
    wl = W.WORKLOADS[W.FWD_TARGET_WORKLOAD]
    inp = W.generate(wl, with_dout=False)
    q, k, v = (dev_tensor(torch, np, getattr(inp, n), wl.dtype) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    B, H, S, D = q.shape
    fws = torch.empty(neox.neox_rope_attn_fwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                      device="cuda")
    n = max(args.steps, 20)
    neox.neox_rope_table_prepare(S, wl.rotary_dim, wl.rope_base)
    call = lambda ev=None: neox.neox_attn_fwd_ex(  # noqa: E731
        q, k, v, o, lse, rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=True,
        softmax_scale=wl.softmax_scale, workspace=fws, phase_events=ev)
    for _ in range(args.warmup):
        call()
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for i in range(n):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    # Split into rotation pass and attention kernel: one reused event set, read
    # after each call (recording many live events slows the host down).
    ev = make_events(torch, 3)
    ms_attn = 0.0
    for i in range(n):
        call(ev)
        torch.cuda.synchronize()
        ms_attn += ev[1].elapsed_time(ev[2])
    ms_attn /= n
    flops = 4 * wl.D * W.total_pairs(inp)
    tf = flops / (ms * 1e-3) / 1e12
    tf_attn = flops / (ms_attn * 1e-3) / 1e12
    return {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "D": wl.D,
            "rotary_dim": wl.rotary_dim, "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "attn_kernel_us": round(ms_attn * 1e3, 2),
            "attn_kernel_frac": round(tf_attn / PEAK_BF16_TFLOPS, 4)}


def fp16_step(args, torch, np, neox, W, wl):
    """The same fwd+bwd step with fp16 storage (the precision FasterTransformer
    runs GPT-NeoX in), timed the same way."""
    import dataclasses
    wl16 = dataclasses.replace(wl, dtype="f16")
    inp16 = W.generate(wl16)
    total_ms, kms = run_gpu(args, torch, np, neox, W, wl16, inp16)
    ms = total_ms / args.steps
    pairs = W.total_pairs(inp16)
    tf = 14 * wl.D * pairs / (ms * 1e-3) / 1e12
    return {"workload": wl.name, "dtype": "f16", "ms_per_step": round(ms, 4), "tflops": round(tf, 2),
            "frac_of_f16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kms.items()}}


def fp8_forward(args, torch, np, neox, W):
    """The FP8 (E4M3) forward at S=2048, D=128 (B=4, H=32, causal), timed back
    to back; algorithmic 4 D flop per allowed pair as for the 16-bit forward."""
    wl = W.FP8_WORKLOADS[W.FP8_BENCH_WORKLOAD]
    inp = W.generate_fp8(wl)
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (inp.q8, inp.k8, inp.v8))
    o = torch.empty((wl.B, wl.H, wl.S, wl.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.B, wl.H, wl.S), dtype=torch.float32, device="cuda")
    call = lambda: neox.neox_attn_fwd_fp8(q8, k8, v8, *inp.scales, o, lse,  # noqa: E731
                                          causal=wl.causal, softmax_scale=wl.softmax_scale)
    for _ in range(max(args.warmup, 2)):
        call()
    n = max(args.steps, 20)
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for _ in range(n):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    flops = 4 * wl.D * wl.B * wl.H * W.allowed_pairs(wl.S, wl.causal)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "D": wl.D,
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def decode(args, torch, np, neox, W):
    """One decoding step (new token against a full 2048-row cache, 20B head
    layout), timed back to back.  Two copies of the cache alternate so that the
    step cannot be served from the last-level cache (each copy is larger than
    it); the rate counts the algorithmic HBM bytes of one step."""
    wl = W.DECODE_WORKLOADS[W.DECODE_BENCH_WORKLOAD]
    inp = W.generate_decode(wl)
    dt = wl.dtype
    q, k, v = (dev_tensor(torch, np, getattr(inp, n), dt) for n in ("q", "k", "v"))
    caches = [(dev_tensor(torch, np, inp.k_cache, dt), dev_tensor(torch, np, inp.v_cache, dt))
              for _ in range(2)]
    lens = torch.from_numpy(inp.lens.copy()).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(neox.neox_rope_attn_decode_workspace_size(wl.B, wl.H, wl.D, wl.cap),
                     dtype=torch.uint8, device="cuda")
    neox.neox_rope_table_prepare(wl.cap, wl.rotary_dim, wl.rope_base)
    call = lambda i: neox.neox_rope_attn_decode(  # noqa: E731
        q, k, v, caches[i & 1][0], caches[i & 1][1], lens, o, lse, wl.rotary_dim, wl.rope_base,
        wl.softmax_scale, workspace=ws)
    for i in range(max(args.warmup, 2)):
        call(i)
    n = max(4 * args.steps, 100)
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for i in range(n):
        call(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    nbytes = W.decode_bytes(wl, inp.lens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": wl.name, "B": wl.B, "H": wl.H, "D": wl.D, "rotary_dim": wl.rotary_dim,
            "cache_rows": wl.cap, "position": int(inp.lens.max()), "us_per_call": round(ms * 1e3, 2),
            "bytes": nbytes, "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("decode", wl.name)}


def cpu_baseline(args, np, W, wl, inp):
    """The oracle (plain float64 numpy) on the first heads of the workload, in
    (b, h) order, until about --cpu-seconds of wall time; rate in TFLOP/s of
    the same algorithmic fwd+bwd work."""
    from oracle import neox_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    slopes = orc.alibi_slopes(wl.H) if wl.alibi else None
    done, flops, t0 = 0, 0, time.perf_counter()
    for b, h in heads:
        sel = lambda n: _head64(W, inp, n, b, h)  # noqa: E731
        offs = None if inp.doc_offsets is None else inp.doc_offsets[b:b + 1]
        orc.attn_bwd(sel("q"), sel("k"), sel("v"), sel("dout"), rotary_dim=wl.rotary_dim,
                     rope_base=wl.rope_base, causal=wl.causal, softmax_scale=wl.softmax_scale,
                     alibi=False if slopes is None else slopes[h:h + 1], doc_offsets=offs)
        pairs = W.allowed_pairs(wl.S, wl.causal, None if offs is None else offs[0])
        flops += 14 * wl.D * pairs
        done += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of {wl.name} (first in (b,h) order), "
                      f"fwd+bwd in float64 numpy, {dt:.1f} s wall"}


def _head64(W, inp, name, b, h):
    import numpy as np
    a = getattr(inp, name)[b:b + 1, h:h + 1]
    if inp.wl.dtype == W.BF16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 (attention "
                                   "heads are independent: N GPUs would each run B*H/N heads "
                                   "with no communication)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import causal_attention_neox_amd as neox
    from causal_attention_neox_amd import _lib
    from causal_attention_neox_amd import workloads as W

    if not os.path.exists(_lib.LIB_PATH):
        from causal_attention_neox_amd.build import build
        build()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.workload or W.BENCH_WORKLOAD]
    inp = W.generate(wl)
    pairs = W.total_pairs(inp)
    fwd_flops = 4 * wl.D * pairs
    bwd_flops = 10 * wl.D * pairs

    total_ms, kms = run_gpu(args, torch, np, neox, W, wl, inp)
    ms_step = total_ms / args.steps
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    rows = wl.B * wl.H * wl.S
    el = 2 if wl.dtype == "bf16" else 4
    kern = {
        "fwd": dict(flops=fwd_flops, ms=kms["fwd"], bound="mfma"),
        # dK/dV pass: S, dP, dV, dK products (8 D flop per allowed pair)
        "bwd_dkdv": dict(flops=8 * wl.D * pairs, ms=kms["bwd_dkdv"], bound="mfma"),
        # dQ pass: the dQ product is its algorithmic work (2 D per pair); it also
        # recomputes S and dP (4 D per pair, reported as "executed")
        "bwd_dq": dict(flops=2 * wl.D * pairs, executed=6 * wl.D * pairs, ms=kms["bwd_dq"],
                       bound="mfma"),
        # q/k rotation pass of the forward: reads q and k, writes the rotated bf16 copies
        "fwd_rope_qk": dict(bytes=2 * rows * wl.D * (el + 2)
                            if wl.rotary_dim > 0 and el == 2 else 0,
                            ms=kms["fwd_rope_qk"], bound="hbm"),
    }
    kern = {n: kd for n, kd in kern.items()
            if kd["ms"] > 0 and (kd["bound"] == "mfma" or kd["bytes"] > 0)}  # passes that ran
    kernels_out = {}
    for name, kd in kern.items():
        sec = kd["ms"] * 1e-3
        if kd["bound"] == "mfma":
            ach = kd["flops"] / sec / 1e12
            kernels_out[name] = {"us": round(kd["ms"] * 1e3, 2), "tflops": round(ach, 1),
                                 "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
            if "executed" in kd:
                kernels_out[name]["executed_tflops"] = round(kd["executed"] / sec / 1e12, 1)
        else:
            ach = kd["bytes"] / sec / 1e9
            kernels_out[name] = {"us": round(kd["ms"] * 1e3, 2), "gbs": round(ach, 1),
                                 "frac": round(ach / PEAK_HBM_GBS, 4)}
    dom = max(kern, key=lambda n: kern[n]["ms"])
    kd = kern[dom]
    if kd["bound"] == "mfma":
        ach = kd["flops"] / (kd["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, wl.name), "kernel": dom}
    else:
        ach = kd["bytes"] / (kd["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom, wl.name),
                "kernel": dom}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "D": wl.D,
                   "rotary_dim": wl.rotary_dim, "rope_base": wl.rope_base, "causal": wl.causal,
                   "alibi": wl.alibi, "packed_docs": wl.packed_docs, "global_batch": wl.B,
                   "seq_len": wl.S, "parallelism": "single-gpu"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "kernels": kernels_out,
    }
    if not args.no_fwd_target:
        out["fwd_target"] = fwd_target(args, torch, np, neox, W)
    if not args.no_fp16:
        out["fp16"] = fp16_step(args, torch, np, neox, W, wl)
    if not args.no_fp8:
        out["fp8_fwd"] = fp8_forward(args, torch, np, neox, W)
    if not args.no_decode:
        out["decode"] = decode(args, torch, np, neox, W)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, np, W, wl, inp)
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        # Known traffic for scaling the HBM byte counters: an elementwise kernel
        # over the whole chip (1 GiB read, 1 GiB written) and the runtime's copy.
        src = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
