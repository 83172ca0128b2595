"""GPU parity of linear verification on batches that take the split path: every row cut
into S slices (2 <= S <= 8), one workgroup each, all resident together.  The B=64, k=5,
V=32000 workload is cut into 2 slices of 512 x 4 per row; the cases below cover 2 to 8
slices and the narrower shapes taken when the wider ones do not fit the chip, every
way a row can end (accepted, rejected with a residual draw, the bonus draw), rows that
reject everywhere or nowhere, k = 0, unaligned bases and draft rows read element-wise,
repeated calls on one workspace (the tagged words of one call must never be taken for
the next call's), and the workspace's status word at zero after every call."""
import numpy as np
import pytest
import torch

import speculative_sampling_verify_03_amd as sv
from gpu_common import announce, check_linear, oracle_linear, run_linear, sections_clear, status_word
from synthetic import cfg2_case, fixed_pq_case, linear_case

pytestmark = pytest.mark.gpu


def _run_checked(case, seed, offset=0, misalign=(0, 0), what=""):
    announce(f"{what}: B={case.B} k={case.k} V={case.V} {case.logits.dtype} misalign={misalign}")
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, case.B, case.k, case.V)
    got = run_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset, misalign,
                     ws=ws)
    assert status_word(ws) == 0, f"{what}: a wait between workgroups ran out"
    assert sections_clear(ws, sv.SV_KIND_LINEAR, case.k, case.V)
    ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset)
    check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=case.V, what=what)
    return got, ref


@pytest.mark.parametrize("case_seed", [2, 102, 202, 302])
def test_headline_batches(case_seed):
    # the four input batches the benchmark rotates through, each with two RNG seeds
    case = cfg2_case(seed=case_seed)
    for seed in (0, 1):
        _run_checked(case, seed, offset=seed, what=f"split B=64 k=5 V=32000 inputs {case_seed} seed {seed}")


@pytest.mark.parametrize("dtype,V,B,k", [
    ("bf16", 8193, 64, 3),     # 2 slices of 256 x 4
    ("bf16", 20001, 64, 4),    # 2 slices of 512 x 4, ragged end
    ("bf16", 65536, 32, 5),    # 192 rows: 5 slices of 256 x 8 (5 x 512 x 4 do not fit)
    ("bf16", 100000, 16, 5),   # 7 slices of 512 x 4
    ("bf16", 32000, 80, 5),    # 480 rows: 512 x 4 and 256 x 4 do not fit, 2 slices of 256 x 8
    ("bf16", 12000, 160, 5),   # 960 rows: 2 slices of 128 x 8 (wider shapes do not fit)
    ("f32", 5000, 48, 4),      # 2 slices of 256 x 4
    ("f32", 16000, 40, 5),     # 2 slices of 512 x 4
    ("f32", 40000, 24, 5),     # 5 slices of 512 x 4
])
def test_slice_counts(dtype, V, B, k):
    case = linear_case(B, k, V, seed=V + B, dtype=dtype, noise_sigma=1.0)
    _run_checked(case, seed=7, what=f"split {dtype} V={V}")


@pytest.mark.parametrize("misalign", [(1, 1), (1, 0), (3, 5)])
def test_unaligned_rows(misalign):
    # odd V: every row starts at a different 16-byte phase; (1, 0) and (3, 5) also put the
    # draft rows out of phase with the logits, so they are read element-wise
    case = linear_case(40, 5, 20001, seed=11, dtype="bf16", noise_sigma=1.0)
    _run_checked(case, seed=3, misalign=misalign, what=f"split unaligned {misalign}")


def test_mixed_dtypes_elementwise_draft_rows():
    case = linear_case(32, 5, 12000, seed=12, dtype="f32", noise_sigma=1.0)
    case.draft_probs = case.draft_probs.to(torch.bfloat16)
    _run_checked(case, seed=6, what="split f32 logits, bf16 draft probs")


def test_every_row_rejects():
    # disjoint supports: position 0 always rejects, every draw is a residual draw from p_0
    V, k = 32000, 5
    p = np.zeros((k + 1, V))
    p[:, :16000] = 1 / 16000
    q = np.zeros((k, V))
    q[:, 16000:] = 1 / 16000
    case = fixed_pq_case(p, q, 64, seed=3, dtype="bf16")
    got, _ = _run_checked(case, seed=8, what="split disjoint supports")
    assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] < 16000)


def test_every_row_accepts():
    # q = p exactly: every draft is kept (outside near-ties) and the bonus comes from p_k
    case = linear_case(64, 5, 32000, seed=13, dtype="f32", noise_sigma=1.0)
    lg = case.logits.double().numpy()
    z = lg[:, :5] - lg[:, :5].max(axis=-1, keepdims=True)
    case.draft_probs = torch.from_numpy(np.exp(z) / np.exp(z).sum(axis=-1, keepdims=True)).to(torch.float32)
    got, ref = _run_checked(case, seed=9, what="split q = p")
    assert np.all(got["accept_len"][~ref["near_tie"]] == 5)


def test_k0_plain_sampling():
    case = linear_case(200, 0, 32000, seed=14, dtype="bf16", noise_sigma=1.0)
    _run_checked(case, seed=10, what="split k=0")


def test_repeated_calls_one_workspace():
    # the slots of one call must not leak into the next, on the same workspace and stream
    case = cfg2_case(seed=2)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, case.B, case.k, case.V)
    ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 4, 0)
    for rep in range(3):
        got = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 4, 0, ws=ws)
        assert status_word(ws) == 0
        check_linear(got, ref, torch.bfloat16, X=case.draft_tokens.numpy(), V=case.V, what=f"split repeat {rep}")


def test_one_workspace_across_sizes_and_kinds():
    # A workspace zero-filled once serves calls of any size and kind in turn: the split
    # kernel's tagged words sit in a prefix whose place never moves, and no later call can
    # take a word left behind for one of its own.
    big = cfg2_case(seed=102)                                           # split, 4 slices
    small = linear_case(10, 3, 32000, seed=15, dtype="bf16", noise_sigma=1.0)  # split, other sizes
    wide = linear_case(16, 5, 70001, seed=16, dtype="bf16", noise_sigma=1.0)   # row kernel (multi-tile)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, 64, 5, 70001)
    for rep in range(2):
        for name, case, seed in (("big", big, 1), ("small", small, 2), ("wide", wide, 3), ("big", big, 4)):
            got = run_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, rep, ws=ws)
            assert status_word(ws) == 0
            ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, rep)
            check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=case.V,
                         what=f"shared workspace {name} pass {rep}")
