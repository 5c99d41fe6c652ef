"""Builds libneoxattn.so (gfx950 kernels + C-ABI host code) in the package
directory with hipcc.  Usable as a module (``build()``) or a script.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled; objects go to ``_build/`` at the repository root and are
linked into ``causal_attention_neox_amd/libneoxattn.so``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libneoxattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # No kernel relies on NaN semantics (masks use -inf, which stays honoured);
    # without NaNs fmaxf needs no operand canonicalisation, which otherwise
    # doubles the row-max instructions of the softmax.
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: a ROCm toolchain with gfx950 support is required")


def sources():
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, n) for n in names]


def _compile(hipcc: str, src: str, obj: str) -> None:
    cmd = [hipcc, *COMMON_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


PROBE_SRC = os.path.join(CSRC, "probe", "mfma_clock.hip")
PROBE_PATH = os.path.join(PKG_DIR, "libneoxprobe.so")


def build_probe(hipcc: str) -> str:
    """The measurement probe (MFMA rate and sustained clock) as its own small
    library; it is no part of libneoxattn."""
    tmp = PROBE_PATH + ".tmp"
    cmd = [hipcc, *COMMON_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def build(jobs: int = 8) -> str:
    """Compiles every source and links the shared library (and the
    measurement probe); returns the library's path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda so: _compile(hipcc, *so), zip(srcs, objs)))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_probe(hipcc)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
