"""Pins of lossless tree verification (oracle/tree_lossless.py).

The page's guarantee ("Speculative decoding explained", section "Draft and verification
loop": the output follows the target distribution exactly) fixes the law of the whole
emitted sequence: token by token it is the target's own autoregressive law, whatever the
tree.  The chi-square test below computes that law from p alone (never from the
verification rule) and compares the oracle's emitted sequences with it; plus special
cases and invariants."""
import numpy as np
from scipy import stats

from oracle import target_distribution, verify_linear, verify_tree_lossless

# BFS order: root 0 with children 1, 2, 3 and 4 (node 4 repeats node 1's token);
# node 1 -> 5, 6; node 2 -> 7, 8; node 3 -> 9 (an invalid token)
PARENTS = [-1, 0, 0, 0, 0, 1, 1, 2, 2, 3]


def _case(V=6, T=0.8, seed=11):
    rng = np.random.default_rng(seed)
    N = len(PARENTS)
    logits = rng.normal(0.0, 1.5, size=(N, V))
    tokens = np.zeros(N, dtype=np.int64)
    # children of the root: its three most likely tokens, then a repeat of the first (node 9)
    top = np.argsort(-logits[0])
    tokens[1], tokens[2], tokens[3], tokens[4] = top[0], top[1], top[2], top[0]
    for u, kids in ((1, (5, 6)), (2, (7, 8)), (3, (9,))):
        t = np.argsort(-logits[u])
        for r, c in enumerate(kids):
            tokens[c] = t[r]
    tokens[9] = V  # an invalid token: never kept
    return logits, tokens, T


def _target_law(logits, tokens, T):
    """Probability of every emitted sequence under the target alone: follow the tree while
    the emitted token is a child's token (the first child carrying it), stop after the
    first token that leaves the tree or after the token drawn below a leaf."""
    N, V = logits.shape
    kids = {u: [c for c in range(1, N) if PARENTS[c] == u] for u in range(N)}
    law = {}

    def walk(u, prefix, prob):
        p = target_distribution(logits[u], T)
        for y in range(V):
            nxt = next((c for c in kids[u] if tokens[c] == y), None)
            if nxt is None:
                law[prefix + (y,)] = prob * p[y]
            else:
                walk(nxt, prefix + (y,), prob * p[y])
    walk(0, (), 1.0)
    return law


def test_emitted_sequence_law_is_the_target_law():
    logits, tokens, T = _case()
    law = _target_law(logits, tokens, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    B = 20000
    L = np.broadcast_to(logits, (B,) + logits.shape)
    X = np.broadcast_to(tokens, (B, len(tokens)))
    r = verify_tree_lossless(L, X, PARENTS, T, seed=5)
    counts = {}
    for b in range(B):
        n = int(r["accept_len"][b])
        key = tuple(int(t) for t in r["tokens"][b, :n + 1])
        counts[key] = counts.get(key, 0) + 1
    assert set(counts) <= set(law)
    keys = sorted(law)
    exp = np.array([law[k] * B for k in keys])
    obs = np.array([counts.get(k, 0) for k in keys], dtype=np.float64)
    # pool the rare outcomes so every cell expects at least 5
    rare = exp < 5
    if rare.any():
        exp = np.append(exp[~rare], exp[rare].sum())
        obs = np.append(obs[~rare], obs[rare].sum())
    _, pval = stats.chisquare(obs, exp)
    assert pval > 1e-4, pval
    # the tree is used: sequences of length 2 and 3 occur
    assert (r["accept_len"] >= 1).mean() > 0.3 and (r["accept_len"] == 2).any()


def test_root_only_is_a_draw_from_p():
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(50, 1, 40))
    r = verify_tree_lossless(logits, np.zeros((50, 1), dtype=np.int64), [-1], 1.3, seed=9)
    lin = verify_linear(logits, np.zeros((50, 0, 40)), np.zeros((50, 0), dtype=np.int64), 1.3, seed=9)
    assert (r["accept_len"] == 0).all()
    assert np.array_equal(r["tokens"][:, 0], lin["tokens"][:, 0])


def test_certain_children_are_always_kept():
    V, N = 8, 5
    parents = [-1, 0, 1, 2, 3]
    logits = np.full((3, N, V), -np.inf)
    tokens = np.array([[0, 3, 5, 1, 7]] * 3)
    for u in range(N - 1):
        logits[:, u, tokens[0, u + 1]] = 0.0        # p concentrated on the child's token
    logits[:, N - 1, :] = 0.0
    r = verify_tree_lossless(logits, tokens, parents, 1.0, seed=1)
    assert (r["accept_len"] == N - 1).all()
    assert np.array_equal(r["tokens"][:, :N - 1], tokens[:, 1:])


def test_rejected_children_are_never_the_extra_token():
    rng = np.random.default_rng(8)
    B, V = 400, 5
    parents = [-1, 0, 0, 0, 1, 1]
    logits = rng.normal(0, 1.0, size=(B, 6, V))
    tokens = np.stack([rng.permutation(V)[:6] if V >= 6 else np.r_[0, rng.permutation(V)] for _ in range(B)])
    r = verify_tree_lossless(logits, tokens, parents, 1.0, seed=2)
    kids = {0: [1, 2, 3], 1: [4, 5]}
    for b in range(B):
        u = int(r["chosen"][b])
        n = int(r["accept_len"][b])
        assert r["path"][b, n] == u
        for d in range(1, n + 1):  # the path follows parent links and emits node tokens
            assert parents[r["path"][b, d]] == r["path"][b, d - 1]
            assert r["tokens"][b, d - 1] == tokens[b, r["path"][b, d]]
        if not r["fallback"][b]:
            assert r["tokens"][b, n] not in [tokens[b, c] for c in kids.get(u, [])]
