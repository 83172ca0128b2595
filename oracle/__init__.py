"""CPU oracle for the speculative verification step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 reference of what the HIP library computes.
Only the test-suite, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the library and its Python binding never do, and this package shares no
code, header, table or constant with them.

Sources (cited by title and section throughout):
  * "Accelerating Sonar through speculation" (Perplexity blog post; read in its Telugu
    and Polish translations) -- called *Sonar* below.
  * "Speculative decoding explained: how any LLM can get 3x faster inference"
    (15jq.com, Hindi) -- called *Explained* below.

Neither page prints a formula.  The readings taken where they are silent (the exact
acceptance comparison, the residual law, the counter-based generator and its counter
layout, tie rules, the tree's bonus rule) are stated next to the code that takes them.

Pinned by tests/test_oracle_*.py against: numpy's independent Philox4x64-10, exact
rational enumeration on tiny vocabularies, chi-square tests of the emitted-token law,
the closed form for the mean emitted length under i.i.d. acceptance, the greedy
identity, the worst and best cases the pages state, and scipy's softmax.  The token plug
is pinned by its invariants (length arithmetic, untouched prefixes, capacity) and by a
multi-step run whose history must equal the concatenated outputs; prompt lookup by
hand-worked histories and by a search with Python's own substring find.  Lossless tree
verification is pinned by a chi-square test of the whole emitted sequence against the
target's own sequence law, which any tree rule that keeps that law must reproduce.
"""
from .philox import philox4x64_10, uniforms  # noqa: F401
from .verify import (  # noqa: F401
    target_distribution,
    inverse_cdf_sample,
    acceptance_overlap,
    verify_linear,
    verify_greedy,
    verify_tree,
    lmhead_logits,
    lmhead_gemm_error_bound,
    lmhead_gemm_error_bound_probabilistic,
    verify_lmhead,
)
from .plug import plug_tokens  # noqa: F401
from .lookup import lookup_drafts  # noqa: F401
from .tree_lossless import verify_tree_lossless  # noqa: F401
