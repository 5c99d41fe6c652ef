"""Writes tests/golden/oracle_small.json: oracle outputs on tiny inputs.

The inputs are built here from a fixed closed-form pattern (no random
generator, nothing from the HIP library); the expected values come only from
oracle/neox_oracle.py.  The file guards the oracle against silent edits; its
correctness rests on the pins in tests/test_oracle_pins.py.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import neox_oracle as orc  # noqa: E402


def pattern(shape, phase):
    n = np.arange(int(np.prod(shape)), dtype=np.float64)
    return np.sin(0.37 * n + phase).reshape(shape) * 1.5


CASES = [
    dict(name="rope_full", B=1, H=2, S=9, D=8, rotary_dim=8, causal=True, alibi=False,
         doc_offsets=None),
    dict(name="rope_partial", B=1, H=1, S=11, D=12, rotary_dim=4, causal=True, alibi=False,
         doc_offsets=None),
    dict(name="alibi_docs", B=2, H=2, S=10, D=4, rotary_dim=0, causal=True, alibi=True,
         doc_offsets=[[0, 3, 10], [0, 10, 10]]),
]


def main():
    out = {"_source": "oracle/neox_oracle.py via tests/golden/make_golden.py", "cases": []}
    for c in CASES:
        shape = (c["B"], c["H"], c["S"], c["D"])
        q, k, v, do = (pattern(shape, ph) for ph in (0.1, 0.7, 1.3, 2.9))
        offs = None if c["doc_offsets"] is None else np.array(c["doc_offsets"], np.int32)
        o, lse, dq, dk, dv = orc.attn_bwd(q, k, v, do, rotary_dim=c["rotary_dim"],
                                          rope_base=100.0, causal=c["causal"],
                                          alibi=c["alibi"], doc_offsets=offs)
        rec = dict(c, rope_base=100.0, q=q.tolist(), k=k.tolist(), v=v.tolist(),
                   dout=do.tolist(), o=o.tolist(), lse=lse.tolist(), dq=dq.tolist(),
                   dk=dk.tolist(), dv=dv.tolist())
        out["cases"].append(rec)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
