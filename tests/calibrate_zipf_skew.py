"""Pick the strength of the rank-1 Zipf component of the skewed 16384-token workload.

Test infrastructure, kept beside the tests rather than in ``oracle/`` because
it reads the package's input recipe: run once by hand, it prints the value
stored as ``ZIPF_BETA`` in ``routing_fp8_grouped_amd/configs.py``.

The skewed workload adds beta * a (x) v to the router centroids, with
a_e = r_e^-1.1 - mean(r^-1.1) over a seeded rank permutation r, so the
affinities follow a Zipf-like profile across experts.  Pure Zipf(1.1) loads are
infeasible (one expert can take at most one slot per token, T of the T*k
slots), so beta is chosen by bisection such that the busiest routed expert gets
about 4000 of the 16384 * 8 slots and the least busy get close to none.  Routing
is the oracle's.

    python -m tests.calibrate_zipf_skew
"""

import dataclasses
import sys

import numpy as np

from oracle.route import route


def counts_for(cfg, beta, x, inputs):
    c = dataclasses.replace(cfg, skew_beta=beta)
    wg = inputs.router_weights(c).float().numpy()
    b = inputs.selection_bias(c).numpy()
    r = route(x, wg, b, c.G, c.M, c.k, c.route_scale)
    return np.bincount(r["idx"].ravel(), minlength=c.E)


def main(target=4000):
    sys.path.insert(0, ".")
    from routing_fp8_grouped_amd import configs, inputs
    cfg = configs.get("zipf_16k")
    x = inputs.activations(cfg).float().numpy()
    lo, hi = 0.0, 8.0
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        cnt = counts_for(cfg, mid, x, inputs)
        print(f"beta={mid:.4f} max={cnt.max()} min={cnt.min()} mean={cnt.mean():.0f}", flush=True)
        if cnt.max() < target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 3)
    cnt = np.sort(counts_for(cfg, beta, x, inputs))[::-1]
    print("beta", beta)
    print("sorted counts (top 16):", cnt[:16].tolist())
    print("sorted counts (bottom 16):", cnt[-16:].tolist())


if __name__ == "__main__":
    main()
