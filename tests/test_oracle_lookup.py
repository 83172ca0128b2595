"""Pins of the prompt-lookup oracle (oracle/lookup.py), "Speculative decoding explained",
section "Variants without a separate draft model": hand-worked histories, and an
independent search that encodes tokens as characters and uses str.find."""
import numpy as np

from oracle import lookup_drafts


def _one(h, mn, mx, k, cap=None):
    cap = cap or len(h) + 3
    H = np.full((1, cap), -9, dtype=np.int64)
    H[0, :len(h)] = h
    d, c = lookup_drafts(H, [len(h)], mn, mx, k)
    return list(d[0]), int(c[0])


def test_hand_worked():
    # "7 8 9" appears at 0; the tokens after it are 1 2 3 7
    assert _one([7, 8, 9, 1, 2, 3, 7, 8, 9], 1, 3, 4) == ([1, 2, 3, 7], 4)
    # the longest phrase wins over a shorter one with another match
    assert _one([5, 9, 1, 2, 9, 6, 1, 2], 1, 2, 2) == ([9, 6], 2)
    # only the last token matches: n = 1 decides (earliest occurrence of 4)
    assert _one([4, 0, 4, 1, 3, 4], 1, 3, 3) == ([0, 4, 1], 3)
    # drafts stop at the end of the history
    assert _one([1, 2, 3, 1, 2], 2, 2, 5) == ([3, 1, 2, -1, -1], 3)
    # no earlier occurrence
    assert _one([1, 2, 3, 4], 1, 2, 3) == ([-1, -1, -1], 0)
    # phrases longer than the history are skipped, not matched against padding
    assert _one([3, 3], 1, 4, 2) == ([3, -1], 1)
    # empty and one-token histories
    assert _one([], 1, 3, 2) == ([-1, -1], 0)
    assert _one([5], 1, 3, 2) == ([-1, -1], 0)


def _by_find(h, mn, mx, k):
    s = "".join(chr(0x4E00 + t) for t in h)   # one character per token
    for n in range(mx, mn - 1, -1):
        if n < 1 or n >= len(h):
            continue
        i = s.find(s[len(h) - n:])
        if 0 <= i < len(h) - n:
            follow = h[i + n:i + n + k]
            return follow + [-1] * (k - len(follow)), len(follow)
    return [-1] * k, 0


def test_matches_substring_find():
    rng = np.random.default_rng(4)
    for trial in range(400):
        L = int(rng.integers(0, 60))
        vocab = int(rng.integers(2, 6))       # small vocabularies: many repeats
        h = [int(t) for t in rng.integers(0, vocab, size=L)]
        mn, mx = int(rng.integers(1, 3)), int(rng.integers(2, 6))
        k = int(rng.integers(1, 8))
        assert _one(h, mn, max(mn, mx), k) == _by_find(h, mn, max(mn, mx), k), (h, mn, mx, k)


def test_invalid_lengths_draft_nothing():
    H = np.array([[1, 2, 1, 2], [1, 2, 1, 2]])
    d, c = lookup_drafts(H, [5, -1], 1, 2, 2)
    assert c.tolist() == [0, 0] and (d == -1).all()
