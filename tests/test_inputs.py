"""CPU checks of the synthetic input recipes: the properties each workload was built to
have still hold for the generators as they stand."""
import numpy as np

from oracle import acceptance_overlap, target_distribution
from synthetic import cfg2_case, to_numpy_f64
from synthetic.generators import CFG2_NOISE_SIGMA


def test_cfg2_noise_sigma_gives_three_quarters_overlap():
    """B=64, k=5, V=32000 bf16: sigma was chosen so that the mean per-position acceptance
    probability sum_v min(p, q) of the seed-2 batch is 0.75, the middle of the 70-80%
    acceptance quoted in "Speculative decoding explained", section "Best and worst case"."""
    case = cfg2_case(seed=2)
    assert case.meta["noise_sigma"] == CFG2_NOISE_SIGMA
    L = to_numpy_f64(case.logits)
    Q = to_numpy_f64(case.draft_probs)
    vals = [acceptance_overlap(target_distribution(L[b, j], 1.0), Q[b, j])
            for b in range(L.shape[0]) for j in range(Q.shape[1])]
    assert abs(float(np.mean(vals)) - 0.75) < 0.005, np.mean(vals)
