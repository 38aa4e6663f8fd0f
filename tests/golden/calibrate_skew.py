"""Calibrate the strength tau of the Zipf router bias of the skewed workload.

Runs only the oracle's router and selection.  Prints, for tau on a 0.05
grid, the number of experts that receive no route and the largest expert
load at 16384 tokens (the 100 lowest-ranked experts switched off), then the
smallest tau whose largest load exceeds 2000.  The chosen value is stored as
workloads.SKEW_TAU.

usage: python tests/golden/calibrate_skew.py
"""
import dataclasses
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def main():
    cfg = W.CONFIGS["skew16k"]
    layer = W.make_layer(cfg, with_experts=False)
    x = W.tokens(cfg)
    base = O.router_logits(x, layer["w_router"])
    chosen = None
    for tau in np.arange(0.05, 3.01, 0.05):
        c = dataclasses.replace(cfg, zipf_tau=float(round(tau, 2)))
        bias = W.zipf_bias(c).astype(np.float64)
        idx = O.select_routes(base + bias[None, :], cfg.top_k)
        load = np.bincount(idx.reshape(-1), minlength=cfg.experts)
        empty, mx = int((load == 0).sum()), int(load.max())
        print(f"tau={tau:.2f} empty={empty} max_load={mx}")
        if chosen is None and mx > 2000:
            chosen = (round(float(tau), 2), empty, mx)
            break
    print("chosen", chosen)


if __name__ == "__main__":
    main()
