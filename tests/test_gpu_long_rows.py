"""Long linear rows (V from 20000 to 262144, walked in tiles by the row kernel: more than
eight slices per row, or more rows than the chip holds in slices, so the split kernel does
not take them) in every dtype pairing, with ragged last tiles, k = 1 over 2200 rows, k = 40,
invalid draft tokens, -inf logits, a residual drawn by every sequence and a residual that
rounding leaves empty, against the oracle."""
import numpy as np
import pytest
import torch

from gpu_common import announce, check_linear, oracle_linear, run_linear, sections_clear, status_word
from synthetic import fixed_pq_case, linear_case

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _run(case, seed, what, ws=None, offset=0, with_probs=True):
    announce(f"{what}: B={case.B} k={case.k} V={case.V} {case.logits.dtype}/{case.draft_probs.dtype} "
             f"T={case.temperature} seed={seed} probabilities={'on' if with_probs else 'off'}")
    got = run_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset, ws=ws,
                     with_probs=with_probs)
    ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset)
    check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=case.V, what=what)
    return got, ref


@pytest.mark.parametrize("lt,qt,V,T", [("bf16", "bf16", 140000, 1.0),  # ragged last unit and chunk
                                       ("bf16", "bf16", 200008, 0.7),
                                       ("f32", "f32", 70000, 1.0),
                                       ("f32", "bf16", 100000, 1.3),
                                       ("bf16", "f32", 262144, 1.0)])  # 64 whole units, 32 chunks
def test_long_rows_dtypes_and_sizes(lt, qt, V, T):
    import speculative_sampling_verify_03_amd as sv
    case = linear_case(48, 4, V, seed=V % 97, dtype=lt, noise_sigma=1.0, temperature=T)
    case.draft_probs = case.draft_probs.to(_DT[qt])
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, case.B, case.k, V)
    for rep in range(2):  # the second call starts from the words the first left
        got, ref = _run(case, 11 + rep, f"long rows {lt}/{qt} V={V} call {rep}", ws=ws, offset=rep)
        assert status_word(ws) == 0
        assert sections_clear(ws, sv.SV_KIND_LINEAR, case.k, V), f"call {rep}: workspace not cleared"
    assert (ref["accept_len"] < case.k).sum() > 0 and (ref["accept_len"] == case.k).sum() > 0


def test_long_rows_single_draft_many_rows():
    # k = 1 with 1100 sequences: 2200 rows of 20000 float32 values
    case = linear_case(1100, 1, 20000, seed=4, dtype="f32", noise_sigma=1.0)
    _run(case, 2, "long rows k=1")


def test_long_rows_long_draft():
    case = linear_case(6, 40, 70000, seed=7, dtype="f32", noise_sigma=0.3)
    _run(case, 5, "long rows k=40")


@pytest.mark.parametrize("B,k,V,lt", [(60, 10, 70000, "f32"), (1100, 1, 20000, "f32"), (260, 8, 40000, "bf16")])
def test_long_rows_tokens_only(B, k, V, lt):
    # no p_j(x_j) outputs: rows after the first rejection stop early (and help it, where
    # the batch allows); two calls on one workspace, which must come back clear
    import speculative_sampling_verify_03_amd as sv
    case = linear_case(B, k, V, seed=B + k, dtype=lt, noise_sigma=0.5 if k > 8 else 1.0)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, B, k, V)
    for rep in range(2):
        _run(case, 21 + rep, f"long rows tokens only B={B} k={k} V={V} call {rep}", ws=ws, offset=rep,
             with_probs=False)
        assert status_word(ws) == 0
        assert sections_clear(ws, sv.SV_KIND_LINEAR, case.k, V), f"call {rep}: workspace not cleared"


@pytest.mark.parametrize("B,k,V,lt,with_probs", [(64, 4, 70000, "bf16", True), (64, 4, 70000, "bf16", False),
                                                 (128, 2, 40000, "f32", True)])
def test_long_rows_last_row_waits(B, k, V, lt, with_probs):
    # one round of workgroups with B k >= 256: each sequence's last row waits for the
    # earlier rows' decisions and streams only when all of them kept their drafts, else it
    # helps the rejected row at once
    import speculative_sampling_verify_03_amd as sv
    case = linear_case(B, k, V, seed=B * k, dtype=lt, noise_sigma=0.7)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, B, k, V)
    for rep in range(2):
        _, ref = _run(case, 31 + rep, f"long rows, last row waits, B={B} k={k} V={V} call {rep}", ws=ws,
                      offset=rep, with_probs=with_probs)
        assert status_word(ws) == 0
        assert sections_clear(ws, sv.SV_KIND_LINEAR, case.k, V), f"call {rep}: workspace not cleared"
    assert (ref["accept_len"] < k).sum() > 0 and (ref["accept_len"] == k).sum() > 0


def test_long_rows_invalid_tokens_and_minus_inf():
    V = 140000
    case = linear_case(16, 4, V, seed=5, dtype="bf16", noise_sigma=1.0)
    case.draft_tokens[:, 1] = torch.tensor([-1, V, 10**6, -(10**6)] * 4, dtype=torch.int32)
    case.logits[:, :, 100000:] = float("-inf")
    got, _ = _run(case, 3, "long rows: invalid tokens and -inf logits")
    assert np.all(got["accept_len"] <= 1)
    emitted = got["tokens"][np.arange(16), got["accept_len"]]
    assert np.all((emitted >= 0) & (emitted < 100000))


def test_long_rows_every_row_rejects():
    # position 0 always rejects (disjoint supports): every sequence draws its residual,
    # which is p_0 itself, over the 32 chunks of a V = 2^18 row
    import speculative_sampling_verify_03_amd as sv
    V, k, B = 1 << 18, 2, 24
    rng = np.random.default_rng(8)
    p = np.zeros((k + 1, V))
    p[:, : V // 2] = rng.uniform(0.5, 1.5, size=(k + 1, V // 2))
    p /= p.sum(axis=1, keepdims=True)
    q = np.zeros((k, V))
    q[:, V // 2:] = rng.uniform(0.5, 1.5, size=(k, V - V // 2))
    q /= q.sum(axis=1, keepdims=True)
    case = fixed_pq_case(p, q, B, seed=6, dtype="f32")
    case.logits = case.logits.to(torch.bfloat16)
    case.draft_probs = case.draft_probs.to(torch.bfloat16)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, B, k, V)
    for rep in range(2):
        got, _ = _run(case, 9, f"long rows residual everywhere call {rep}", ws=ws, offset=rep)
        assert sections_clear(ws, sv.SV_KIND_LINEAR, k, V)
        assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] < V // 2)


def test_long_rows_empty_residual_draws_from_p():
    # p and q put all their mass on one token, and the draft token is another one (q(x) =
    # p(x) = 0): the test rejects it and max(0, p - q) is zero everywhere, so the emitted
    # token is drawn from p itself: the one token
    V, k, B = 70000, 3, 32
    p = np.zeros((k + 1, V))
    q = np.zeros((k, V))
    hot = [17, 69999, 8192, 5]
    for j in range(k + 1):
        p[j, hot[j]] = 1.0
    for j in range(k):
        q[j, hot[j]] = 1.0
    case = fixed_pq_case(p, q, B, seed=1, dtype="f32")
    case.draft_tokens[:] = torch.tensor([100, 200, 300], dtype=torch.int32)
    got, ref = _run(case, 4, "long rows: empty residual")
    assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] == hot[0])
    assert np.all(ref["tokens"][:, 0] == hot[0])
