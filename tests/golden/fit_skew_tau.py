"""Fit tau of the skewed workload's logit bias b_e = -tau * ln(rank_e).

Target: the most loaded expert receives 15x the mean load (T*k/E) under the
oracle's router, on an 8192-token sample of the skewed workload drawn on the
CPU.  Load is monotone in tau, so bisection finds it.  The printed value is
the constant SKEW_TAU of sparse_moe_layer_wave_amd/inputs.py.

Run from the repository root:  python tests/golden/fit_skew_tau.py
"""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle                                          # noqa: E402
from sparse_moe_layer_wave_amd import inputs           # noqa: E402

TARGET = 15.0


def hot_ratio(x_bits, W, rank, tau, k, scale):
    bias = (-tau * np.log(rank)).astype(np.float32)
    r = oracle.route(x_bits, W, k, scale, bias)
    E = W.shape[0]
    load = np.bincount(r.idx.reshape(-1), minlength=E)
    return load.max() / (x_bits.shape[0] * k / E), load


def main():
    c = inputs.CONFIGS["hy3_long_skewed_T65536"]
    T = 8192
    x = inputs.bits(inputs.make_x(T, c["d"], c["seed"], "cpu"))
    W, _ = inputs.make_router(c["E"], c["d"], c["seed"], "cpu", skew=False)
    W = W.numpy()
    gb = inputs._gen("cpu", c["seed"], inputs._STREAM_BIAS)
    rank = (torch.randperm(c["E"], generator=gb).to(torch.float64) + 1.0).numpy()
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        ratio, _ = hot_ratio(x, W, rank, mid, c["k"], inputs.ROUTER_SCALE)
        if ratio < TARGET:
            lo = mid
        else:
            hi = mid
    tau = round(0.5 * (lo + hi), 4)
    ratio, load = hot_ratio(x, W, rank, tau, c["k"], inputs.ROUTER_SCALE)
    top = np.sort(load)[::-1][:5] / (T * c["k"] / c["E"])
    print(f"tau={tau} hottest/mean={ratio:.2f} top5/mean={np.round(top, 2).tolist()}")


if __name__ == "__main__":
    main()
