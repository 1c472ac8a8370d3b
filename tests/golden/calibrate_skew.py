"""Calibrate the Zipf bias scale of the skewed 8K workload (run once, by hand).

Bisects beta so that, routed by the CPU oracle on the seed-0 draw, the hottest
expert receives 10x the mean load T*k/E.  The printed beta, rounded to a
multiple of 1/1024, is the SKEW_BETA constant in workloads.py; the test
test_oracle_pins.py::test_skew_calibration re-checks the 10 +- 0.5 ratio.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402
import workloads as W  # noqa: E402


def hot_ratio(beta: float) -> float:
    wl = W.get("skewed_8k")
    idx, _ = oracle.route(W.gen_logits(wl, beta), wl.G, wl.g, wl.k)
    load = np.bincount(idx.ravel(), minlength=wl.E)
    return load.max() / (wl.T * wl.k / wl.E)


def main():
    lo, hi = 0.0, 1.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if hot_ratio(mid) < 10.0:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi) * 1024) / 1024
    print(f"beta = {beta!r}  ratio = {hot_ratio(beta):.3f}")


if __name__ == "__main__":
    main()
