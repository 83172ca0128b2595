"""Find the target-noise sigma of the B=64, k=5, V=32000 bf16 workload.

Bisects sigma so that the mean over all (sequence, draft position) pairs of the
acceptance probability sum_v min(p, q) -- p the target distribution of the bf16
logits, q the bf16 draft probabilities -- is 0.75, the middle of the 70-80% acceptance
quoted by "Speculative decoding explained" (section "Best and worst case").  The result
is written by hand into synthetic/generators.py as CFG2_NOISE_SIGMA.

Run:  python -m oracle.tune_cfg2_sigma
"""
from __future__ import annotations

import numpy as np

from synthetic.generators import linear_case, to_numpy_f64
from .verify import acceptance_overlap, target_distribution


def mean_overlap(sigma: float, seed: int = 2) -> float:
    case = linear_case(64, 5, 32000, seed=seed, dtype="bf16", draft_sigma=3.0,
                       noise_sigma=sigma, boost_frac=0.05, boost=8.0)
    L = to_numpy_f64(case.logits)
    Q = to_numpy_f64(case.draft_probs)
    vals = [acceptance_overlap(target_distribution(L[b, j], 1.0), Q[b, j])
            for b in range(L.shape[0]) for j in range(Q.shape[1])]
    return float(np.mean(vals))


def main(target: float = 0.75, lo: float = 0.3, hi: float = 1.2, steps: int = 12):
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        a = mean_overlap(mid)
        print(f"sigma={mid:.10f} mean_overlap={a:.5f}", flush=True)
        if a > target:
            lo = mid
        else:
            hi = mid
    print(f"sigma={0.5 * (lo + hi):.10f}")


if __name__ == "__main__":
    main()
