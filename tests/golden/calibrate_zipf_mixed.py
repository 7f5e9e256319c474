"""Calibrate the router-bias exponent s of the DeepSeek-V3-shaped mixed batch.

The workload asks for a skewed router bias giving routed max/mean of about 1.5 over the
experts.  With the bias family b[e] = -s * ln(e + 1), this script bisects s on the oracle's
routing of the workload's own seeded inputs and writes tests/golden/zipf_mixed.json.
It calls only oracle/ and the input generator.

    python tests/golden/calibrate_zipf_mixed.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402

TARGET = 1.5


def max_to_mean(w, s):
    x = mi.host_tensor_f32(w, "x")
    wr = mi.host_tensor_f32(w, "w_router")
    L = oracle.router_logits(x, wr, mi.zipf_bias(w.E, s))
    idx = oracle.select_topk(L, w.k)
    n = np.bincount(idx.reshape(-1), minlength=w.E)
    return oracle.expert_stats(n, w.T, w.k)["expert_max_to_mean"]


def main():
    w = mi.WORKLOADS["dsv3_mixed"]
    lo, hi = 0.0, 0.2
    assert max_to_mean(w, lo) < TARGET < max_to_mean(w, hi)
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if max_to_mean(w, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    s = round(hi, 6)
    r = max_to_mean(w, s)
    out = {"workload": w.name, "bias": "b[e] = -s * ln(e + 1)", "target_max_to_mean": TARGET,
           "s": s, "routed_max_to_mean": r}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_mixed.json")
    json.dump(out, open(path, "w"), indent=1)
    print(out)


if __name__ == "__main__":
    main()
