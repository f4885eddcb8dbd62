"""Writes tests/golden/oracle_small.json from the oracle alone.

The stored values guard the oracle's arithmetic against silent change: a
later edit that alters any of them must name, in its commit message, the
passage of the pages (or the reading of it) that justifies the change.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")


def cases():
    res = {}
    for fmt, name in ((W.FMT_NVFP4, "nvfp4"), (W.FMT_Q4_0, "q4_0")):
        r = W.streams(100 + fmt)
        w = W.rand_weight(fmt, r["codes"], r["scales"], 24, 160)
        x = W.rand_bf16(r["x"], (5, 160))
        y, b = oracle.gemm(w, x, nthreads=1)
        res["gemm_" + name] = {"y_hex": [float(v).hex() for v in y.reshape(-1)],
                               "b_hex": [float(v).hex() for v in b.reshape(-1)]}
    r = W.streams(120)
    z = r["x"].standard_normal((6, 40)).astype(np.float32)
    q = W.rand_dirichlet_rows(r["q"], 5, 40, 0.5)
    for trial in range(8):
        d = r["drafts"].integers(0, 40, 5).astype(np.int32)
        u = W.rand_uniforms(r["uniforms"], 6)
        tg = oracle.accept_greedy(z, d, 11)
        tr = oracle.accept_rejection(z, q, d, u, 0.6, 0.95, 11)
        res["accept_%d" % trial] = {"greedy": [tg[0].tolist(), tg[1].tolist(), tg[2]],
                                    "rejection": [tr[0].tolist(), tr[1].tolist(), tr[2]]}
    return res


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(cases(), f, indent=0, sort_keys=True)
    print("wrote", OUT)
