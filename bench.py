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
efficiency at S=2048, D=128, per-workload legs (median per-call forward,
backward and fwd+bwd times of every workload: the fp32 S=128 case as HBM GB/s,
the others as TFLOP/s), the HBM rate of the forward at S = 128, 256, 512, the
measured MFMA rate and sustained clock, the same step with fp16 storage, the
FP8 forward at S=2048, D=128, the decoding step's HBM rate (one new token per
sequence against a 2048-row cache), rocprofv3 counter summaries of the
benchmark kernels (when taken from the current sources), and the CPU oracle
timed on a bounded sample of the same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import gc
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
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="workload name (default: the 20B layout)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-fwd-target", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the per-workload legs")
    ap.add_argument("--no-small-s", action="store_true", help="skip the small-S HBM sweep")
    ap.add_argument("--no-probe", action="store_true", help="skip the MFMA rate / clock probe")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with kernels of known traffic (scale for traffic counters)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="no GPU work: summarise the rocprofv3 CSVs under DIR (trace/, sq/, "
                         "fetch/, write/ from the commands in profiles/counters.json) into "
                         "profiles/counters.json")
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
    """HBM bytes per launch of `kernel` on `workload` from profiles/counters.json
    (FETCH_SIZE and WRITE_SIZE counters scaled by a plain copy), or None when
    absent or when the kernel's sources changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            ent = json.load(f)["kernels"][f"{workload}/{kernel}"]
        if source_digest(ent["sources"]) != ent["sources_sha256"]:
            return None
        return int(ent["summary"]["fetch_bytes"] + ent["summary"]["write_bytes"])
    except (OSError, KeyError, ValueError, TypeError):
        return None


# ---------------------------------------------------------------- profile summary

FWD_SOURCES = ["causal_attention_neox_amd/csrc/fwd_bf16.hip",
               "causal_attention_neox_amd/csrc/device_common.hpp",
               "causal_attention_neox_amd/csrc/kernels.hpp"]
BWD_SOURCES = ["causal_attention_neox_amd/csrc/bwd_bf16.hip",
               "causal_attention_neox_amd/csrc/device_common.hpp",
               "causal_attention_neox_amd/csrc/kernels.hpp"]
# (workload, kernel key, pattern of the kernel symbol, sources) of the kernels
# the profile covers: the benchmark step (D=96) and the S=2048, D=128 forward.
PROFILE_KERNELS = [
    ("neox20b_s2048_h64_d96_rd24", "fwd_rope_qk", "rope_qk_kernel<96", FWD_SOURCES),
    ("neox20b_s2048_h64_d96_rd24", "fwd", "fwd_bf16_kernel<96,", FWD_SOURCES),
    ("neox20b_s2048_h64_d96_rd24", "bwd_dq", "bwd_dq_kernel<96,", BWD_SOURCES),
    ("neox20b_s2048_h64_d96_rd24", "bwd_dkdv", "bwd_dkdv_kernel<96,", BWD_SOURCES),
    ("rope_s2048_d128", "fwd_rope_qk", "rope_qk_kernel<128", FWD_SOURCES),
    ("rope_s2048_d128", "fwd", "fwd_bf16_kernel<128,", FWD_SOURCES),
]
# Counter passes serialise every dispatch: a few steps suffice.  The kernel
# trace runs the benchmark's own step count so that its averages compare with
# the live per-kernel times the same command prints.
PROFILE_PROGRAM = ("python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-legs "
                   "--no-small-s --no-probe --no-fp16 --no-fp8 --no-decode --copy-calibration")
PROFILE_TRACE_PROGRAM = ("python3 $REPO/bench.py --no-cpu-baseline --no-legs --no-small-s "
                         "--no-probe --no-fp16 --no-fp8 --no-decode")
PROFILE_PASSES = {
    "trace": "--kernel-trace --stats",
    "sq": "--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_BANK_CONFLICT "
          "SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAVES GRBM_GUI_ACTIVE",
    "fetch": "--pmc FETCH_SIZE TCC_EA0_RDREQ_DRAM_sum",
    "write": "--pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum",
}
N_CU, N_SIMD, N_XCD = 256, 1024, 8


def _csv_rows(pattern):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_profile(d):
    """profiles/counters.json from the CSVs of the passes in PROFILE_PASSES.

    Derived figures (per dispatch, then averaged over the dispatches of the
    kernel): GRBM_GUI_ACTIVE is reported summed over the 8 XCDs, so one XCD's
    active cycles are its eighth; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (that
    x 1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / (that x 256 CUs);
    occupancy = 4 SQ_WAVE_CYCLES / (that x 256 CUs x 32 wave slots);
    LDS bank conflicts per access = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE
    - SQ_LDS_BANK_CONFLICT) and as a share of LDS-busy cycles; HBM bytes =
    FETCH_SIZE and WRITE_SIZE (KiB) scaled by what they read for torch.neg
    over 2^28 fp32 (1 GiB read, 1 GiB written) in the same run."""
    import re
    import statistics as st
    out = {"_about": summarize_profile.__doc__.strip(), "commands": {}, "kernels": {}}
    for name, opts in PROFILE_PASSES.items():
        prog = PROFILE_TRACE_PROGRAM if name == "trace" else PROFILE_PROGRAM
        out["commands"][name] = (f"cd /tmp && TMPDIR=/tmp rocprofv3 {opts} --output-format csv "
                                 f"-d <out>/{name} -o p -- {prog}")
    trace = _csv_rows(os.path.join(d, "trace", "**", "*kernel_trace.csv"))
    pmc = {n: _csv_rows(os.path.join(d, n, "**", "*counter_collection.csv"))
           for n in ("sq", "fetch", "write")}

    def per_dispatch(rows, pat):
        disp = {}
        for r in rows:
            if pat(r["Kernel_Name"]):
                disp.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = \
                    float(r["Counter_Value"])
        return list(disp.values())

    neg = lambda k: "neg_kernel" in k or ("elementwise" in k and "neg" in k)  # noqa: E731
    cal = {}
    for n, c in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        vals = [dd[c] for dd in per_dispatch(pmc[n], neg) if c in dd]
        cal[n] = vals[-1] if vals else None
    out["copy_calibration"] = {"kernel": "torch.neg, 2^28 fp32 (1 GiB read, 1 GiB written)",
                               "fetch_kib_raw": cal["fetch"], "write_kib_raw": cal["write"]}
    gib_kib = float(1 << 20)
    for wl, key, sym, srcs in PROFILE_KERNELS:
        pat = lambda k, sym=sym: sym.replace(" ", "") in k.replace(" ", "")  # noqa: E731
        durs = []
        for r in trace:
            if pat(r.get("Kernel_Name", "")):
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        sq = per_dispatch(pmc["sq"], pat)
        fe = per_dispatch(pmc["fetch"], pat)
        wr = per_dispatch(pmc["write"], pat)
        if not (durs or sq or fe or wr):
            continue
        summ = {}
        if durs:
            summ.update(trace_dispatches=len(durs), avg_us=round(st.mean(durs), 2),
                        min_us=round(min(durs), 2), max_us=round(max(durs), 2),
                        median_us=round(st.median(durs), 2))
        if sq:
            def mean_of(f):
                return st.mean(f(x) for x in sq)
            xcd = lambda x: x["GRBM_GUI_ACTIVE"] / N_XCD  # noqa: E731
            summ["mfma_busy_pct"] = round(100 * mean_of(
                lambda x: x["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd(x) * N_SIMD)), 2)
            summ["valu_busy_pct"] = round(100 * mean_of(
                lambda x: x["SQ_ACTIVE_INST_VALU"] / (xcd(x) * N_CU)), 2)
            summ["occupancy_pct"] = round(100 * mean_of(
                lambda x: 4 * x["SQ_WAVE_CYCLES"] / (xcd(x) * N_CU * 32)), 2)
            summ["lds_bank_conflicts_per_access"] = round(mean_of(
                lambda x: x["SQ_LDS_BANK_CONFLICT"] /
                max(x["SQ_LDS_IDX_ACTIVE"] - x["SQ_LDS_BANK_CONFLICT"], 1.0)), 5)
            summ["lds_bank_conflict_cycles_pct_of_lds_active"] = round(100 * mean_of(
                lambda x: x["SQ_LDS_BANK_CONFLICT"] / max(x["SQ_LDS_IDX_ACTIVE"], 1.0)), 3)
            summ["waves"] = round(mean_of(lambda x: x["SQ_WAVES"]))
            summ["pmc_dispatches"] = len(sq)
        if fe and cal["fetch"]:
            kib = st.mean(x["FETCH_SIZE"] for x in fe)
            summ["fetch_bytes"] = int(kib / cal["fetch"] * gib_kib * 1024)
            summ["fetch_kib_raw"] = round(kib, 3)
            summ["tcc_ea_rdreq_dram"] = round(st.mean(x.get("TCC_EA0_RDREQ_DRAM_sum", 0.0)
                                                      for x in fe))
        if wr and cal["write"]:
            kib = st.mean(x["WRITE_SIZE"] for x in wr)
            summ["write_bytes"] = int(kib / cal["write"] * gib_kib * 1024)
            summ["write_kib_raw"] = round(kib, 3)
            h = st.mean(x.get("TCC_HIT_sum", 0.0) for x in wr)
            m = st.mean(x.get("TCC_MISS_sum", 0.0) for x in wr)
            summ["l2_hit_pct"] = round(100 * h / max(h + m, 1.0), 2)
        if "fetch_bytes" in summ and "avg_us" in summ:
            summ["fetch_tb_per_s_at_avg_us"] = round(summ["fetch_bytes"] / summ["avg_us"] / 1e6, 2)
        sym_seen = sorted({r["Kernel_Name"] for r in pmc["sq"] + trace
                           if pat(r.get("Kernel_Name", ""))})
        out["kernels"][f"{wl}/{key}"] = {
            "workload": wl, "kernel": key,
            "symbol": (re.search(r"\w+_kernel(<[^()]*>)?", sym_seen[0]).group(0)
                       if sym_seen else sym),
            "sources": srcs, "sources_sha256": source_digest(srcs), "summary": summ}
    path = os.path.join(ROOT, "profiles", "counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v["summary"] for k, v in out["kernels"].items()}, indent=1))
    return path


def measured_counters(workload):
    """rocprofv3 counter summary per kernel of `workload` from
    profiles/counters.json, keeping only kernels whose sources are unchanged
    since the counters were taken (None when nothing is left)."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    out = {}
    for name, ent in data.get("kernels", {}).items():
        try:
            if ent["workload"] == workload and \
                    source_digest(ent["sources"]) == ent["sources_sha256"]:
                out[name] = ent["summary"]
        except (OSError, KeyError):
            continue
    return out or None


def per_call_ms(torch, fn, n, warmup):
    """Per-call times of n back-to-back calls of fn() (each between two events
    on the current stream): (median, mean) in ms."""
    for _ in range(warmup):
        fn()
    evs = [make_events(torch, 2) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return t[len(t) // 2], sum(t) / len(t)


def fwd_bytes(wl, out_el=None):
    """Algorithmic HBM bytes of one forward call: q, k, v read once, o and lse
    written once."""
    el = 4 if wl.dtype == "f32" else 2
    rows = wl.B * wl.H * wl.S
    return rows * wl.D * (3 * el + (out_el or el)) + rows * 4


# Every workload the library is checked on, timed on its own (the fwd+bwd
# legs) -- the fp32 S=128 case is forward-only and latency/HBM bound.
LEG_WORKLOADS = ["fp32_s128_d64", "bf16_s2048_d64_rd16", "neox20b_s2048_h64_d96_rd24",
                 "long_s16384_d128", "alibi_docs_s4096_d128", "rope_s2048_d128"]


def workload_leg(args, torch, np, neox, W, wl, inp):
    """Median per-call forward, backward and fwd+bwd times of one workload
    through the _ex calls (the forward's workspace feeds the backward, as in a
    training step)."""
    q, k, v = (dev_tensor(torch, np, getattr(inp, n), wl.dtype) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    B, H, S, D = q.shape
    docs = None if inp.doc_offsets is None else torch.from_numpy(inp.doc_offsets).cuda()
    pos = neox.NEOX_POS_ALIBI if wl.alibi else neox.NEOX_POS_ROPE
    kw = dict(pos=pos, rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
              softmax_scale=wl.softmax_scale, doc_offsets=docs)
    neox.neox_rope_table_prepare(S, wl.rotary_dim, wl.rope_base)
    size = (neox.neox_rope_attn_bwd_workspace_size if wl.backward
            else neox.neox_rope_attn_fwd_workspace_size)(B, H, S, D)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    pairs = W.total_pairs(inp)
    n = max(args.steps, 20)
    fwd = lambda: neox.neox_attn_fwd_ex(q, k, v, o, lse, workspace=ws, **kw)  # noqa: E731
    f_med, f_mean = per_call_ms(torch, fwd, n, args.warmup)
    res = {"B": B, "H": H, "S": S, "D": D, "rotary_dim": wl.rotary_dim, "dtype": wl.dtype,
           "alibi": wl.alibi, "packed_docs": wl.packed_docs, "pairs": pairs,
           "fwd_us": round(f_med * 1e3, 2), "fwd_us_mean": round(f_mean * 1e3, 2),
           "fwd_tflops": round(4 * D * pairs / (f_med * 1e-3) / 1e12, 2)}
    res["fwd_frac"] = round(res["fwd_tflops"] / PEAK_BF16_TFLOPS, 4)
    nb = fwd_bytes(wl)
    res["fwd_bytes"] = nb
    res["fwd_gbs"] = round(nb / (f_med * 1e-3) / 1e9, 1)
    if not wl.backward:
        res["fwd_hbm_frac"] = round(res["fwd_gbs"] / PEAK_HBM_GBS, 4)
        return res
    do = dev_tensor(torch, np, inp.dout, wl.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bwd = lambda: neox.neox_attn_bwd_ex(q, k, v, o, do, lse, dq, dk, dv,  # noqa: E731
                                        workspace=ws, reuse_rotated_qk=True, **kw)
    fwd()
    b_med, b_mean = per_call_ms(torch, bwd, n, args.warmup)

    def step():
        fwd()
        bwd()

    s_med, s_mean = per_call_ms(torch, step, n, args.warmup)
    res.update({"bwd_us": round(b_med * 1e3, 2), "bwd_us_mean": round(b_mean * 1e3, 2),
                "bwd_tflops": round(10 * D * pairs / (b_med * 1e-3) / 1e12, 2),
                "step_us": round(s_med * 1e3, 2), "step_us_mean": round(s_mean * 1e3, 2),
                "step_tflops": round(14 * D * pairs / (s_med * 1e-3) / 1e12, 2)})
    res["bwd_frac"] = round(res["bwd_tflops"] / PEAK_BF16_TFLOPS, 4)
    res["step_frac"] = round(res["step_tflops"] / PEAK_BF16_TFLOPS, 4)
    return res


def workload_legs(args, torch, np, neox, W):
    out = {}
    for name in LEG_WORKLOADS:
        wl = W.WORKLOADS[name]
        inp = W.generate(wl)
        out[name] = workload_leg(args, torch, np, neox, W, wl, inp)
        del inp
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def small_s_sweep(args, torch, np, neox, W):
    """The forward at S = 128, 256, 512 with the B*H and D of the S=2048, D=128
    shape (B=4, H=32, full rotary, bf16): few pairs per byte, so reported as the
    HBM rate of the algorithmic bytes, for the call with a workspace (rotation
    pass, then the rotation-free kernel: the faster form) and without one (the
    kernel rotates q and k as it loads them)."""
    base = W.WORKLOADS[W.FWD_TARGET_WORKLOAD]
    out = []
    for S in (128, 256, 512):
        wl = base.with_sizes(name=f"{base.name}_s{S}", S=S)
        inp = W.generate(wl, with_dout=False)
        q, k, v = (dev_tensor(torch, np, getattr(inp, n), wl.dtype) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        neox.neox_rope_table_prepare(S, wl.rotary_dim, wl.rope_base)
        fws = torch.empty(neox.neox_rope_attn_fwd_workspace_size(wl.B, wl.H, S, wl.D),
                          dtype=torch.uint8, device="cuda")
        t = {}
        for tag, w in (("ws", fws), ("no_ws", None)):
            fwd = lambda w=w: neox.neox_attn_fwd_ex(  # noqa: E731
                q, k, v, o, lse, rotary_dim=wl.rotary_dim, rope_base=wl.rope_base,
                softmax_scale=wl.softmax_scale, workspace=w)
            t[tag] = per_call_ms(torch, fwd, max(4 * args.steps, 100), args.warmup)
        med, mean = t["ws"]
        nb = fwd_bytes(wl)
        gbs = nb / (med * 1e-3) / 1e9
        out.append({"B": wl.B, "H": wl.H, "S": S, "D": wl.D, "us": round(med * 1e3, 2),
                    "us_mean": round(mean * 1e3, 2), "bytes": nb, "gbs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                    "tflops": round(4 * wl.D * W.total_pairs(inp) / (med * 1e-3) / 1e12, 2),
                    "us_no_workspace": round(t["no_ws"][0] * 1e3, 2),
                    "gbs_no_workspace": round(nb / (t["no_ws"][0] * 1e-3) / 1e9, 1)})
    return out


def mfma_probe(args, torch):
    """Dense bf16 MFMA rate of a kernel that issues nothing else (2048
    workgroups of 4 waves, 8 independent 32x32x16 chains per wave) and the
    shader clock the SIMDs ran at meanwhile (s_memtime ticks over the 100 MHz
    s_memrealtime ticks, median over workgroups)."""
    import ctypes
    path = os.path.join(ROOT, "causal_attention_neox_amd", "libneoxprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.neoxprobe_mfma_flops.restype = ctypes.c_double
    lib.neoxprobe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.neoxprobe_mfma_launch.restype = ctypes.c_int
    lib.neoxprobe_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    grid, iters = 2048, 4000
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: lib.neoxprobe_mfma_launch(grid, iters, ctypes.c_void_p(out.data_ptr()),  # noqa
                                             ctypes.c_void_p(clk.data_ptr()), stream)
    if call() != 0:
        return None
    med, _ = per_call_ms(torch, call, 5, 1)
    ticks = clk.view(grid, 2).cpu().numpy().astype("float64")
    ghz = sorted(ticks[:, 0] / ticks[:, 1] * 0.1)
    tf = lib.neoxprobe_mfma_flops(grid, iters) / (med * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(0)
    return {"tflops": round(tf, 1), "frac_of_published_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "clock_ghz_median": round(ghz[len(ghz) // 2], 3), "clock_ghz_min": round(ghz[0], 3),
            "clock_ghz_max": round(ghz[-1], 3),
            "published_peak_tflops": round(PEAK_BF16_TFLOPS, 1),
            "peak_at_measured_clock_tflops": round(256 * 4096 * ghz[len(ghz) // 2] / 1e3, 1),
            "cus": int(getattr(props, "multi_processor_count", 0)),
            "us": round(med * 1e3, 2)}


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
        neox.neox_attn_fwd_ex(q, k, v, o, lse, workspace=ws,
                              phase_events=None if ev is None else ev[0:3], **kw)
        neox.neox_attn_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, workspace=ws,
                              phase_events=None if ev is None else ev[3:7],
                              reuse_rotated_qk=True, **kw)

    for _ in range(args.warmup):
        step(None)
    # Phase events (per-kernel times) on every `stride`-th step of the timed
    # steps: recording seven live events per step can make the host, not the
    # GPU, set the pace of the loop.
    stride = max(1, args.steps // 10)
    events = {s: make_events(torch, 7) for s in range(0, args.steps, stride)}
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(events.get(s))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    def avg(i, j):
        return sum(ev[i].elapsed_time(ev[j]) for ev in events.values()) / len(events)

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
    for _ in range(max(args.warmup, 200)):  # ~40 ms: the clocks settle at the load
        call()
    # n back-to-back calls, three times; the split into rotation pass and
    # attention kernel comes from phase events on every `stride`-th call (a
    # distinct event set each, so the calls stay in their steady state).  The
    # fastest of the three runs is reported: on these GPUs a run of identical
    # calls now and then takes several times longer with the GPU idle between
    # kernels, which is no property of the kernels.
    stride = max(1, n // 10)
    runs = []
    for _ in range(3):
        evs = {i: make_events(torch, 3) for i in range(0, n, stride)}
        start, end = make_events(torch, 2)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            call(evs.get(i))
        end.record()
        torch.cuda.synchronize()
        runs.append((start.elapsed_time(end) / n,
                     sum(ev[1].elapsed_time(ev[2]) for ev in evs.values()) / len(evs)))
    ms, ms_attn = min(runs)
    flops = 4 * wl.D * W.total_pairs(inp)
    tf = flops / (ms * 1e-3) / 1e12
    tf_attn = flops / (ms_attn * 1e-3) / 1e12
    return {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "D": wl.D,
            "rotary_dim": wl.rotary_dim, "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "attn_kernel_us": round(ms_attn * 1e3, 2),
            "attn_kernel_frac": round(tf_attn / PEAK_BF16_TFLOPS, 4),
            "runs_us_per_call": [round(r[0] * 1e3, 2) for r in runs]}


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


def host_cpu():
    """(nproc, CPU model) of this host."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    model = None
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:  # pragma: no cover
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return nproc, model


def cpu_baseline(args, np, W, wl, inp):
    """The oracle (plain float64 numpy) on the first heads of the workload, in
    (b, h) order, until about --cpu-seconds of wall time: per head the forward
    alone, then the forward+backward definition; rates in TFLOP/s of the same
    algorithmic work (4 D flop per pair forward, 10 D backward = the second
    call's time less the first's)."""
    from oracle import neox_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    nproc, model = host_cpu()
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    slopes = orc.alibi_slopes(wl.H) if wl.alibi else None
    done, pairs_done, t_fwd, t_all = 0, 0, 0.0, 0.0
    t0 = time.perf_counter()
    for b, h in heads:
        sel = lambda n: _head64(W, inp, n, b, h)  # noqa: E731
        offs = None if inp.doc_offsets is None else inp.doc_offsets[b:b + 1]
        kw = dict(rotary_dim=wl.rotary_dim, rope_base=wl.rope_base, causal=wl.causal,
                  softmax_scale=wl.softmax_scale,
                  alibi=False if slopes is None else slopes[h:h + 1], doc_offsets=offs)
        q, k, v, do = sel("q"), sel("k"), sel("v"), sel("dout")
        ta = time.perf_counter()
        orc.attn_fwd(q, k, v, **kw)
        tb = time.perf_counter()
        orc.attn_bwd(q, k, v, do, **kw)
        tc = time.perf_counter()
        t_fwd += tb - ta
        t_all += tc - tb
        pairs_done += W.allowed_pairs(wl.S, wl.causal, None if offs is None else offs[0])
        done += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    D = wl.D
    return {"value": round(14 * D * pairs_done / t_all / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of {wl.name} (first in (b,h) order): "
                      f"forward alone {t_fwd:.1f} s, then fwd+bwd {t_all:.1f} s, float64 numpy",
            "nproc": nproc, "cpu_model": model, "threads_used": cores,
            "fwd_gflops": round(4 * D * pairs_done / t_fwd / 1e9, 3),
            "bwd_gflops": round(10 * D * pairs_done / max(t_all - t_fwd, 1e-9) / 1e9, 3),
            "fwd_bwd_gflops": round(14 * D * pairs_done / t_all / 1e9, 3),
            "fwd_s_per_head": round(t_fwd / done, 4),
            "fwd_bwd_s_per_head": round(t_all / done, 4)}


def _head64(W, inp, name, b, h):
    import numpy as np
    a = getattr(inp, name)[b:b + 1, h:h + 1]
    if inp.wl.dtype == W.BF16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
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

    # No cyclic garbage collection while GPU work is being issued: a full
    # collection can hold the issuing thread for milliseconds, and the GPU
    # then idles inside a timed region.
    gc.disable()
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
    if not args.no_probe:
        out["mfma_probe"] = mfma_probe(args, torch)
        if out["mfma_probe"]:
            out["roofline"]["frac_of_measured_peak"] = round(
                roof["achieved"] / out["mfma_probe"]["tflops"], 4) if roof["bound"] == "mfma" \
                else None
    out["counters"] = measured_counters(wl.name)
    if not args.no_fwd_target:
        out["fwd_target"] = fwd_target(args, torch, np, neox, W)
        out["fwd_target"]["counters"] = measured_counters(W.FWD_TARGET_WORKLOAD)
    if not args.no_legs:
        out["workloads"] = workload_legs(args, torch, np, neox, W)
    if not args.no_small_s:
        out["small_s_hbm"] = small_s_sweep(args, torch, np, neox, W)
    if not args.no_fp16:
        out["fp16"] = fp16_step(args, torch, np, neox, W, wl)
    if not args.no_fp8:
        out["fp8_fwd"] = fp8_forward(args, torch, np, neox, W)
    if not args.no_decode:
        out["decode"] = decode(args, torch, np, neox, W)
    gc.enable()
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
