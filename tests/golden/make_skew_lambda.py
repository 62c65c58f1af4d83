"""Calibrate the skewed-routing bias scale with the oracle's routing.

The skewed workload's correction bias is lam * log p_e with Zipf(s=1.2)
popularity p_e ~ (e+1)^-1.2.  This script bisects lam on the seeded inputs
until exactly round(0.2 * n_routed) experts receive no token, then rounds lam
to 3 significant digits (keeping the count) and writes
tests/golden/skew_lambda.json.  It calls only the oracle and the input
generator.  Run from the repository root:

    python tests/golden/make_skew_lambda.py
"""
import dataclasses
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mixture_experts_feed_amd import workloads as wl  # noqa: E402


def empty_experts(w, z, lam):
    w2 = dataclasses.replace(w, bias_dist=("zipf", w.bias_dist[1], lam))
    b = wl.correction_bias(w2).double().numpy()
    _, idx, _, _ = oracle.route(z, b, w.n_routed, w.top_k, w.route_scale, w.global_scale)
    counts, _, _ = oracle.permutation(idx, w.n_routed)
    return int((counts == 0).sum()), counts


def main():
    w = wl.WORKLOADS["skewed_h6144"]
    target = int(round(0.2 * w.n_routed))
    x = wl.hidden_states(w).float().numpy()
    z = oracle.gate_logits(x, wl.gate_bank(w).numpy())
    lo, hi = 0.0, 1.0          # empty(lo) < target <= empty(hi)
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        n, _ = empty_experts(w, z, mid)
        if n >= target:
            hi = mid
        else:
            lo = mid
    # shortest decimal in [lo, hi] giving the target count
    lam = hi
    for digits in range(2, 8):
        cand = float(f"{hi:.{digits}g}")
        if empty_experts(w, z, cand)[0] == target:
            lam = cand
            break
    n, counts = empty_experts(w, z, lam)
    res = dict(workload=w.name, target_empty=target, lam=lam, empty=n,
               max_count=int(counts.max()), min_nonempty=int(counts[counts > 0].min()))
    print(json.dumps(res))
    with open(os.path.join(ROOT, "tests", "golden", "skew_lambda.json"), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
