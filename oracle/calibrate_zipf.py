"""Calibrates the Zipf bias strength of the two skewed-load workloads.

The skewed workload is described by two targets that the logit-bias model
(seeded N(0,1) logits + beta * (-1.2 * ln rank_e)) cannot meet at once: the 8
most popular experts taking ~40% of the T*k assignments, and ~30 experts
receiving none.  Each target gets its own workload, calibrated here by a
deterministic bisection on beta under the workload's own routing (oracle
routing of the seeded logits):
  skew        -- beta at which the top-8 share reaches 40%;
  skew-empty  -- the smallest beta (to 1e-6) at which at least 30 experts are empty.
Prints beta, the realised top-8 share and the number of empty experts for each;
the printed betas are the values stored in synth.CONFIGS.  Calls only oracle/
and synth/.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import synth  # noqa: E402


def load(cfg, beta):
    ids, _ = oracle.route_cfg(cfg, synth.logits(cfg, beta=beta))
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    top8 = np.sort(counts)[::-1][:8].sum() / ids.size
    return top8, int(np.sum(counts == 0))


def bisect(cfg, reached):
    """Smallest beta in [0, 4] (to 2^-40 of the range) at which reached(top8, empty) holds."""
    lo, hi = 0.0, 4.0
    for _ in range(40):
        mid = (lo + hi) / 2
        if reached(*load(cfg, mid)):
            hi = mid
        else:
            lo = mid
    return hi


def main():
    for name, reached in (("skew", lambda top8, empty: top8 >= 0.40),
                          ("skew-empty", lambda top8, empty: empty >= 30)):
        cfg = synth.CONFIGS[name]
        beta = round(bisect(cfg, reached), 6)
        if not reached(*load(cfg, beta)):  # rounding to 6 digits stepped below the threshold
            beta = round(beta + 1e-6, 6)
        s, empty = load(cfg, beta)
        print(f"{name}: beta={beta} top8_share={s:.4f} empty_experts={empty}")


if __name__ == "__main__":
    main()
