"""MI355X (gfx950) speculative verification library: linear speculative sampling, greedy
and static-tree verification (plus a lossless tree variant), and an LM-head projection feeding verification, behind a
small C ABI (include/spec_verify.h), plus an on-device token plug for the next step and
prompt-lookup drafting.  This package is the thin Python binding over it."""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SV_BF16,
    SV_F32,
    SV_KIND_GREEDY,
    SV_KIND_LINEAR,
    SV_KIND_LMHEAD,
    SV_KIND_TREE,
    SpecVerifyError,
    library,
    new_workspace,
    spec_lmhead_logits,
    spec_lmhead_verify,
    spec_verify_linear_noalloc,
    spec_lookup_drafts,
    spec_plug_tokens,
    spec_verify_greedy,
    spec_verify_linear,
    spec_verify_strerror,
    spec_verify_tree,
    spec_verify_tree_lossless,
    spec_verify_workspace_bytes,
)
