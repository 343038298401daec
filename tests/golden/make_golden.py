"""Write tests/golden/oracle_small.json: the oracle's outputs on one tiny seeded case.

Calls only oracle/ (and the seeded input generator).  The pages print no numeric
worked example for these kernels (TensorFold PR #1169 "Receipt" reports only
pass/fail of the page suite and served timings), so the stored values here are
the oracle's own, kept to catch unintended changes to its arithmetic: any later
change to them must name, in its commit message, the passage or reading that
justifies it.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from paged_kv_cache_pg_amd.inputs import make_workload  # noqa: E402

CASE = dict(seed=5, lens=[13, 8], page_pos=4, n_q_heads=4, n_kv_heads=2, head_dim=8, dtype="bf16",
            table_kind="shuffled", idx_dim=8, n_idx_heads=2)


def compute():
    w = make_workload(**CASE)
    q, K, V, IK, qI = (w.as_f64(n) for n in ("q", "K", "V", "IK", "qI"))
    scale = 1 / np.sqrt(8)
    dec = O.decode(q, K, V, w.lens, scale)
    pooled = O.pool(IK, w.lens)
    sc = [O.scores(qI[s], pooled[s]) for s in range(2)]
    top = [O.topk(sc[s], 2) for s in range(2)]
    sp = O.sparse(q, K, V, top, scale)
    pre = O.prefill(q[:1].reshape(1, 4, 8).repeat(3, axis=0), K[0], V[0], 10, scale)
    return {
        "case": CASE,
        "scale": scale,
        "decode": dec.tolist(),
        "pooled": [p.astype(np.float64).tolist() for p in pooled],
        "scores": [s.tolist() for s in sc],
        "topk2": [t.tolist() for t in top],
        "sparse": sp.tolist(),
        "prefill_q0x3_at10": pre.tolist(),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(compute(), f, indent=1)
