"""Calibrate the Zipf popularity bias strength and store it for the generators.

TEST INFRASTRUCTURE ONLY.  Run:  python -m oracle.calibrate_zipf
Writes fixtures/zipf_beta.json.

The skewed workloads bias every expert's router logit by -beta * 1.1 * ln(r_e)
(r_e its popularity rank, Zipf exponent s = 1.1).  beta is bisected on the
workload's own seeded tokens until the ceil(0.1 E) most-picked experts receive
50 % (+- 1 %) of the unrestricted top-k assignments ("the top 10% of experts
receive about 50% of assignments").  Routing here is the oracle's (O1, O3).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import fixtures
from oracle import moe

TARGET, TOL = 0.50, 0.01


def top_share(z0: np.ndarray, ranks: np.ndarray, beta: float, k: int) -> float:
    E = z0.shape[1]
    b = fixtures.zipf_bias(ranks, beta).astype(np.float64)
    picks = moe.topk(z0 + b[None, :], k)
    counts = np.bincount(picks.reshape(-1), minlength=E)
    top = np.sort(counts)[::-1][:math.ceil(0.1 * E)]
    return float(top.sum() / picks.size)


def calibrate(name: str) -> dict:
    lay = fixtures.make_layer(name, beta=0.0)
    cfg = lay.cfg
    z0 = moe.router_logits(lay.x_bits, lay.w_router, None)
    ranks = lay.ranks
    lo, hi = 0.0, 4.0
    beta, share = None, None
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        share = top_share(z0, ranks, mid, cfg.k)
        beta = mid
        if abs(share - TARGET) <= TOL / 4:
            break
        if share < TARGET:
            lo = mid
        else:
            hi = mid
    assert abs(share - TARGET) <= TOL, (name, beta, share)
    return {"beta": round(beta, 6), "top10_share": round(share, 6), "tokens": int(cfg.T),
            "workload": name}


def main():
    out = {"prefill": calibrate("prefill"), "long": calibrate("long")}
    path = os.path.join(os.path.dirname(fixtures.__file__), "zipf_beta.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
