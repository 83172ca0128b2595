"""GPU parity of the on-device token plug (spec_plug_tokens) against oracle/plug.py:
bit-exact lengths, histories, next tokens and status codes, on random verify outputs, on
capacity and invalid-input edges, and chained after real verification calls."""
import numpy as np
import pytest
import torch

import speculative_sampling_verify_03_amd as sv
from gpu_common import announce, check_linear, oracle_linear, run_linear
from oracle import plug_tokens
from synthetic import linear_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_plug(toks, n, lens, hist):
    t = torch.as_tensor(np.asarray(toks), dtype=torch.int32, device=DEV).contiguous()
    a = torch.as_tensor(np.asarray(n), dtype=torch.int32, device=DEV).contiguous()
    L = torch.as_tensor(np.asarray(lens), dtype=torch.int32, device=DEV).contiguous()
    H = torch.as_tensor(np.asarray(hist), dtype=torch.int32, device=DEV).contiguous()
    nxt = torch.full((t.shape[0],), -1, dtype=torch.int32, device=DEV)
    st = torch.full((t.shape[0],), -5, dtype=torch.int32, device=DEV)
    sv.spec_plug_tokens(t, a, L, H, nxt, st)
    torch.cuda.synchronize()
    return L.cpu().numpy(), H.cpu().numpy(), nxt.cpu().numpy(), st.cpu().numpy()


def _compare(got, ref, what):
    gl, gh, gn, gs = got
    rl, rh, rn, rs = ref
    assert np.array_equal(gl, rl), f"{what}: lengths"
    assert np.array_equal(gh, rh), f"{what}: histories"
    assert np.array_equal(gs, rs), f"{what}: status"
    ok = rs != 2   # next_token is not written for invalid rows
    assert np.array_equal(gn[ok], rn[ok]), f"{what}: next tokens"
    assert (gn[~ok] == -1).all()


@pytest.mark.parametrize("B,W,cap", [(1, 1, 1), (37, 6, 50), (1000, 9, 300), (300, 64, 100), (5, 64, 2)])
def test_plug_random(B, W, cap):
    announce(f"plug random B={B} W={W} cap={cap}")
    rng = np.random.default_rng(B * 131 + W)
    n = rng.integers(0, W, size=B)
    toks = np.full((B, W), -1, dtype=np.int64)
    for b in range(B):
        toks[b, :n[b] + 1] = rng.integers(0, 128256, size=n[b] + 1)
    lens = rng.integers(0, cap + 1, size=B)
    hist = rng.integers(0, 1000, size=(B, cap))
    _compare(_gpu_plug(toks, n, lens, hist), plug_tokens(toks, n, lens, hist), f"B={B} W={W} cap={cap}")


def test_plug_invalid_rows():
    announce("plug invalid accept lengths and lengths")
    toks = np.array([[5, 6, -1], [7, -1, -1], [8, 9, 10], [1, 2, 3]])
    n = np.array([3, -1, 0, 1])
    lens = np.array([0, 0, 5, 4])
    hist = np.arange(16).reshape(4, 4)
    _compare(_gpu_plug(toks, n, lens, hist), plug_tokens(toks, n, lens, hist), "invalid rows")


def test_plug_empty_batch():
    announce("plug B=0")
    t = torch.empty((0, 6), dtype=torch.int32, device=DEV)
    a = torch.empty((0,), dtype=torch.int32, device=DEV)
    sv.spec_plug_tokens(t, a, a.clone(), torch.empty((0, 10), dtype=torch.int32, device=DEV))


def test_plug_chained_after_verification():
    """Eight decoding steps: GPU verify -> GPU plug, against oracle verify -> oracle plug.
    A sequence whose verification hits a near-tie (where both results are valid but may
    differ) is dropped from the comparison from then on."""
    announce("plug chained after linear verification, 8 steps")
    B, k, V, cap = 48, 5, 4000, 64
    lens_g = torch.zeros(B, dtype=torch.int32, device=DEV)
    hist_g = torch.full((B, cap), -3, dtype=torch.int32, device=DEV)
    nxt_g = torch.empty(B, dtype=torch.int32, device=DEV)
    lens_r = np.zeros(B, dtype=np.int64)
    hist_r = np.full((B, cap), -3, dtype=np.int64)
    tracked = np.ones(B, dtype=bool)
    for s in range(8):
        c = linear_case(B, k, V, seed=500 + s, dtype="bf16", noise_sigma=0.6)
        got = run_linear(c.logits, c.draft_probs, c.draft_tokens, 1.0, 11, offset=s)
        ref = oracle_linear(c.logits, c.draft_probs, c.draft_tokens, 1.0, 11, offset=s)
        check_linear(got, ref, torch.bfloat16, c.draft_tokens.numpy(), V, what=f"chained step {s}")
        differs = (got["tokens"] != ref["tokens"]).any(axis=1) | (got["accept_len"] != ref["accept_len"])
        tracked &= ~(ref["near_tie"].astype(bool) & differs)
        toks = torch.as_tensor(got["tokens"], dtype=torch.int32, device=DEV)
        alen = torch.as_tensor(got["accept_len"], dtype=torch.int32, device=DEV)
        sv.spec_plug_tokens(toks, alen, lens_g, hist_g, nxt_g)
        lens_r, hist_r, nxt_r, _ = plug_tokens(ref["tokens"], ref["accept_len"], lens_r, hist_r)
        torch.cuda.synchronize()
        t = tracked
        assert np.array_equal(lens_g.cpu().numpy()[t], lens_r[t]), f"step {s}: lengths"
        assert np.array_equal(hist_g.cpu().numpy()[t], hist_r[t]), f"step {s}: histories"
        assert np.array_equal(nxt_g.cpu().numpy()[t], nxt_r[t]), f"step {s}: next tokens"
    assert tracked.sum() >= B - 4
