"""Writes tests/golden/tiny_seed0.json by calling only the CPU oracle.

The pages print no worked example, so this fixture is a regression record of
the oracle itself on the tiny workload (1 sequence, 4 heads, d 64, 1024 tokens,
exact-score top-k 32, sinks 4, window 32, eps = delta = 0.05, seed 0).  Any
later change to the oracle's arithmetic that moves these values must name the
passage or reading that justifies it.
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic  # noqa: E402


def record():
    w = synthetic.tiny(seed=0)
    r = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_dense=True)
    heads = []
    for h in range(w.Hq):
        idx = r["idx"][0, h]
        idx = idx[idx >= 0]
        heads.append(dict(counts=[int(x) for x in r["counts"][0, h]],
                          stats=[str(int(x)) for x in r["stats"][0, h]],
                          idx_sha1=hashlib.sha1(idx.astype("<i4").tobytes()).hexdigest(),
                          idx_head=[int(x) for x in idx[:16]],
                          lse=float(r["lse"][0, h]), lse_dense=float(r["lse_dense"][0, h]),
                          out_l2=float(np.linalg.norm(r["out"][0, h]))))
    return dict(workload="tiny_1k", seed=0, z32=r["z32"], heads=heads)


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(record(), f, indent=1)
