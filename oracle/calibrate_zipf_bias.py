"""Writes the per-rank logit bias of the skewed-routing workload.

Test infrastructure: run by hand (``python -m oracle.calibrate_zipf_bias``);
its output, ``sparse_mixture_experts_kept_amd/data/zipf_bias.json``, is a
constant of the input recipe.  It uses the oracle's own top-2 selection so the
bias is calibrated against the routing rule the layer follows.

Target: expert of rank r (1..8) receives a share of the token slots
proportional to r^-1.2 (Zipf, s = 1.2).  Scores without bias are modelled as
iid N(0, 1.28^2), the spread of x W_g^T for an RMS-normalised x and router
weights of std 0.02 at d = 4096.  Iteration: b <- b + 0.7 log(p_target /
p_realised), re-centred to mean 0, 60 times, on 400,000 fixed-seed rows.
"""

import json
import os

import numpy as np

from oracle.moe_oracle import select_top_k

S = 1.2
E = 8
ROWS = 400_000
ITERS = 60
STEP = 0.7
SIGMA = 1.28


def target_shares():
    w = np.arange(1, E + 1, dtype=np.float64) ** -S
    return w / w.sum()


def realised_shares(logits):
    idx = select_top_k(logits, 2)
    return np.bincount(idx.reshape(-1), minlength=E) / idx.size


def main():
    rng = np.random.default_rng(20240108)
    base = rng.standard_normal((ROWS, E)) * SIGMA
    p = target_shares()
    b = np.zeros(E)
    for _ in range(ITERS):
        q = realised_shares(base + b)
        b = b + STEP * np.log(p / q)
        b -= b.mean()
    q = realised_shares(base + b)
    out = {
        "description": "per-rank logit bias for the Zipf(s=1.2) skewed-routing workload (rank 1 = hottest)",
        "writer": "oracle/calibrate_zipf_bias.py",
        "s": S, "sigma": SIGMA, "rows": ROWS, "iters": ITERS, "step": STEP,
        "target_shares": p.tolist(),
        "realised_shares": q.tolist(),
        "bias_by_rank": b.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "sparse_mixture_experts_kept_amd", "data", "zipf_bias.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
