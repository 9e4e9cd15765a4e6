"""One-off search for the smoothing widths of the locality-plus-sink generator.

Runs the oracle's mask steps only (pooling, pooled softmax, hybrid selection) on the 720p
token grid at the workload's own k_frac and p, for sigma_(y,x) in {2, 4, 8, 16, 24, 32, 48}
and sigma_t in {1, 2, 4} (by default), and prints the realised kept-block density of each setting. The first
setting inside [4%, 6%] is the one to freeze in ``configs.CALIBRATED_SIGMA``; k_frac and p are
never touched. Usage: ``python -m workloads.calibrate [--heads 8]``.
"""

from __future__ import annotations

import argparse
import math
from dataclasses import replace

import numpy as np

import oracle
from .configs import WORKLOADS
from .gen import make_inputs


def density(w, heads) -> float:
    kept = 0
    total = 0
    for h in heads:
        x = make_inputs(w, heads=[h])
        q = x["q"].to(dtype=x["q"].dtype).float().numpy()
        k = x["k"].float().numpy()
        mask, _ = oracle.block_mask(q, k, w.bq, w.bk, w.k_frac, w.p, 1.0 / math.sqrt(w.head_dim))
        kept += int(mask.sum())
        total += mask.size
    return kept / total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="wan720p")
    ap.add_argument("--heads", type=int, default=8)
    ap.add_argument("--sigma-yx", type=float, nargs="+", default=[2.0, 4.0, 8.0, 16.0, 24.0, 32.0, 48.0])
    ap.add_argument("--sigma-t", type=float, nargs="+", default=[1.0, 2.0, 4.0])
    args = ap.parse_args()
    base = WORKLOADS[args.workload]
    heads = list(range(args.heads))
    for s_yx in args.sigma_yx:
        for s_t in args.sigma_t:
            w = replace(base, sigma=(s_t, s_yx, s_yx))
            dens = density(w, heads)
            flag = "  <- in [4%, 6%]" if 0.04 <= dens <= 0.06 else ""
            print(f"sigma_t={s_t:g} sigma_yx={s_yx:g} density={100 * dens:.2f}%{flag}", flush=True)


if __name__ == "__main__":
    main()
