"""Calibrate the strength of the Zipf logit offset of the 40-layer skewed workload.

TEST INFRASTRUCTURE: writes ``tests/golden/zipf_alpha.json``, which the input
generator reads.  Only the oracle's arithmetic is used (numpy float64 router
products and the oracle's top-k selection).

Workload: 40 stacked layers, T=4096, each layer's router logits offset by
``-alpha * 1.1 * ln(rank(e))`` with a seeded popularity ranking, ``alpha`` set
so that the 16 most-used experts of a layer receive half of the token-expert
assignments (mean over the 40 layers).  Bisection on alpha over the seeded
data with the activations as first drawn (attempt 0).

Run:  python -m oracle.calibrate_zipf
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import moe_synth  # noqa: E402
import oracle  # noqa: E402
from oracle.tie_filter import router_logits_f64  # noqa: E402

TARGET = 0.50
TOP = 16


def top_share(idx, E, top=TOP):
    counts = np.bincount(idx.ravel(), minlength=E)
    return np.sort(counts)[::-1][:top].sum() / idx.size


def mean_share(base_logits, ranks, alpha, k, E):
    shares = []
    for l, r in zip(base_logits, ranks):
        bias = (-alpha * moe_synth.ZIPF_S * np.log(r.astype(np.float64))).astype(np.float32)
        idx, _ = oracle.select(l + bias.astype(np.float64)[None, :], k)
        shares.append(top_share(idx, E))
    return float(np.mean(shares))


def main():
    cfg = moe_synth.CONFIGS["stack40"]
    E, k = cfg.shape.E, cfg.shape.top_k
    x = moe_synth.token_rows(cfg)
    base = [router_logits_f64(x, moe_synth.router_weights(cfg, l)) for l in range(cfg.layers)]
    ranks = [moe_synth.zipf_ranks(cfg, l) for l in range(cfg.layers)]
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if mean_share(base, ranks, mid, k, E) < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 6)
    share = mean_share(base, ranks, alpha, k, E)
    out = {
        "alpha": alpha,
        "zipf_s": moe_synth.ZIPF_S,
        "top": TOP,
        "mean_top16_share_attempt0": round(share, 5),
        "written_by": "oracle/calibrate_zipf.py",
        "workload": "40 layers, T=4096, E=256, top-8, seed 4",
    }
    with open(moe_synth.ZIPF_ALPHA_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
