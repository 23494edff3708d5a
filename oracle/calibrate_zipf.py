"""Calibrates the Zipf bias strength of the skewed-load workload.

Deterministic bisection on beta so that, under the workload's own routing
(oracle routing of the seeded logits N(0,1) + beta * (-1.2 * ln rank_e)), the
8 most popular experts receive 40% of the T*k assignments.  Prints beta, the
realised top-8 share and the number of empty experts; the printed beta is the
value stored in synth.CONFIGS["skew"].  Calls only oracle/ and synth/.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import synth  # noqa: E402


def share(cfg, beta):
    ids, _ = oracle.route_cfg(cfg, synth.logits(cfg, beta=beta))
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    top8 = np.sort(counts)[::-1][:8].sum() / ids.size
    return top8, int(np.sum(counts == 0))


def main():
    cfg = synth.CONFIGS["skew"]
    lo, hi = 0.0, 4.0
    for _ in range(40):
        mid = (lo + hi) / 2
        s, _ = share(cfg, mid)
        if s < 0.40:
            lo = mid
        else:
            hi = mid
    beta = round((lo + hi) / 2, 6)
    s, empty = share(cfg, beta)
    print(f"beta={beta} top8_share={s:.4f} empty_experts={empty}")


if __name__ == "__main__":
    main()
