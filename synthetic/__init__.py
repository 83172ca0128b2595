"""Seeded synthetic inputs for the speculative verification step.

This package only *makes inputs*: draft and target logits, draft probabilities, draft
tokens, static trees, LM-head weights and hidden states.  It holds none of the
verification arithmetic (no target softmax, no acceptance test, no residual, no
sampler of emitted tokens, no random-number generator of the method).  Both the HIP
path and the CPU oracle consume what it returns.
"""
from .generators import (  # noqa: F401
    Case,
    TreeCase,
    LMHeadCase,
    linear_case,
    cfg1_case,
    cfg2_case,
    cfg3_case,
    cfg4_case,
    cfg5_case,
    mtp_case,
    lookup_histories,
    tree_case,
    lmhead_case,
    eagle_tree_parents,
    chain_tree_parents,
    fixed_pq_case,
    to_numpy_f64,
    CFG2_NOISE_SIGMA,
)
