"""Pins of the token-plug oracle (oracle/plug.py), "Accelerating Sonar through speculation",
section "MTP schedule for one token".  The operation is an append, so it is pinned by what
an append must satisfy rather than by retyping it: lengths add up, prefixes are untouched,
the capacity is respected, invalid inputs change nothing, and over several verification
steps the history equals the emitted tokens concatenated with Python lists."""
import numpy as np
import pytest

from oracle import plug_tokens, verify_linear
from synthetic import linear_case, to_numpy_f64


def _random_outputs(rng, B, W):
    n = rng.integers(0, W, size=B)
    toks = np.full((B, W), -1, dtype=np.int64)
    for b in range(B):
        toks[b, :n[b] + 1] = rng.integers(0, 50000, size=n[b] + 1)
    return toks, n


def test_invariants_random():
    rng = np.random.default_rng(0)
    B, W, cap = 200, 6, 40
    toks, n = _random_outputs(rng, B, W)
    lens = rng.integers(0, cap + 1, size=B)
    hist = rng.integers(0, 1000, size=(B, cap))
    new_len, new_hist, nxt, status = plug_tokens(toks, n, lens, hist)
    for b in range(B):
        end = lens[b] + n[b] + 1
        assert new_len[b] == min(end, cap)
        assert status[b] == (1 if end > cap else 0)
        assert nxt[b] == toks[b, n[b]]
        assert np.array_equal(new_hist[b, :lens[b]], hist[b, :lens[b]])           # prefix kept
        kept = min(end, cap) - lens[b]
        assert list(new_hist[b, lens[b]:lens[b] + kept]) == list(toks[b, :kept])  # appended
        assert np.array_equal(new_hist[b, lens[b] + kept:], hist[b, lens[b] + kept:])
    # the inputs are not modified
    assert hist.shape == (B, cap)


def test_invalid_inputs_change_nothing():
    toks = np.array([[5, 6, -1], [7, -1, -1], [8, 9, 10]])
    hist = np.zeros((3, 4), dtype=np.int64)
    new_len, new_hist, nxt, status = plug_tokens(toks, [3, -1, 0], [0, 0, 5], hist)
    assert list(status) == [2, 2, 2]
    assert list(new_len) == [0, 0, 5]
    assert not new_hist.any()
    assert list(nxt) == [-1, -1, -1]


def test_exact_fill_and_overflow():
    toks = np.array([[1, 2, 3], [4, 5, 6]])
    hist = np.zeros((2, 5), dtype=np.int64)
    new_len, new_hist, nxt, status = plug_tokens(toks, [2, 2], [2, 3], hist)
    assert list(new_len) == [5, 5] and list(status) == [0, 1]
    assert list(new_hist[0]) == [0, 0, 1, 2, 3]
    assert list(new_hist[1]) == [0, 0, 0, 4, 5]     # token 6 dropped at the capacity
    assert list(nxt) == [3, 6]


def test_history_is_the_concatenated_outputs_over_steps():
    B, k, V, cap, steps = 12, 4, 300, 64, 6
    hist = np.full((B, cap), -7, dtype=np.int64)
    lens = np.zeros(B, dtype=np.int64)
    emitted = [[] for _ in range(B)]
    for s in range(steps):
        c = linear_case(B, k, V, seed=100 + s, dtype="f32", noise_sigma=0.8)
        r = verify_linear(to_numpy_f64(c.logits), to_numpy_f64(c.draft_probs), c.draft_tokens.numpy(), 1.0, 7, s)
        toks, n = r["tokens"], r["accept_len"]
        for b in range(B):
            emitted[b] += [int(t) for t in toks[b, :n[b] + 1]]
        lens, hist, nxt, status = plug_tokens(toks, n, lens, hist)
        assert not status.any()
    for b in range(B):
        assert int(lens[b]) == len(emitted[b])
        assert [int(t) for t in hist[b, :lens[b]]] == emitted[b]
        assert (hist[b, lens[b]:] == -7).all()
