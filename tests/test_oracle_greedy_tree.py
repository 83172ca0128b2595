"""Pins of the oracle's greedy and static-tree verification.

Greedy: identical draft and target with argmax drafts always emit k+1 tokens; ties take
the lowest index; the first mismatch stops the run.
Tree ("Accelerating Sonar through speculation", section "EAGLE"): the chosen node is
re-derived by enumerating every root-to-leaf path with acceptance bits recomputed here
from scipy's softmax and the Philox draws; the exact law of the chosen node on a tiny
tree is enumerated over all acceptance outcomes and compared with the oracle's
frequencies; a chain tree reduces to counting consecutive acceptances.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import uniforms, verify_greedy, verify_tree
from oracle.verify import tree_depths
from synthetic import (chain_tree_parents, eagle_tree_parents, linear_case, to_numpy_f64,
                       tree_case)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


@pytest.mark.parametrize("k", [1, 4, 8])
def test_greedy_identity_emits_k_plus_one(k):
    case = linear_case(40, k, 300, seed=k, dtype="bf16")
    L = to_numpy_f64(case.logits)
    X = np.argmax(L[:, :k], axis=-1)  # draft = target, greedy drafting
    out = verify_greedy(L, X)
    assert np.all(out["accept_len"] == k)
    assert np.all(out["tokens"][:, :k] == X)
    assert np.all(out["tokens"][:, k] == np.argmax(L[:, k], axis=-1))


def test_greedy_ties_take_lowest_index_and_stop_at_mismatch():
    V = 10
    L = np.zeros((3, 4, V))
    L[:, :, [2, 5, 7]] = 4.0  # three-way tie
    X = np.array([[2, 2, 2], [2, 5, 2], [7, 2, 2]])
    out = verify_greedy(L, X)
    assert np.all(out["argmax"] == 2)
    assert list(out["accept_len"]) == [3, 1, 0]
    assert list(out["tokens"][1]) == [2, 2, -1, -1]
    assert list(out["tokens"][2]) == [2, -1, -1, -1]


def test_greedy_vs_python_max():
    case = linear_case(30, 5, 64, seed=9, dtype="bf16", noise_sigma=0.3)
    L = to_numpy_f64(case.logits)
    X = case.greedy_tokens.numpy()
    out = verify_greedy(L, X)
    for b in range(30):
        g = [max(range(64), key=lambda v: (L[b, j, v], -v)) for j in range(6)]
        n = next((j for j in range(5) if g[j] != X[b, j]), 5)
        assert out["accept_len"][b] == n
        assert out["tokens"][b, n] == g[n]


def test_eagle_tree_shape_matches_page_facts():
    facts = json.load(open(GOLDEN))["eagle_static_tree"]
    par = eagle_tree_parents(tuple(facts["branching"]), facts["nodes"])
    assert par.shape[0] == facts["nodes"]
    assert int(tree_depths(par).max()) == facts["max_accept_len"]
    assert par[0] == -1 and np.all(par[1:] < np.arange(1, par.shape[0]))
    assert np.all(np.diff(par[1:]) >= 0)


def _paths(par):
    N = len(par)
    children = [[c for c in range(1, N) if par[c] == u] for u in range(N)]
    out = []

    def rec(u, path):
        if not children[u]:
            out.append(path)
        for c in children[u]:
            rec(c, path + [c])
    rec(0, [0])
    return out


@pytest.mark.parametrize("branching,V,seed", [((4, 2, 2, 2), 200, 0), ((3, 3, 1), 50, 1),
                                              ((2, 2, 2, 2, 2), 30, 2)])
def test_tree_choice_by_path_enumeration(branching, V, seed):
    par = eagle_tree_parents(branching, 64)
    case = tree_case(60, par, V, seed=seed, dtype="bf16", noise_sigma=1.0,
                     sample_children=(seed % 2 == 1))
    L = to_numpy_f64(case.logits)
    Q = to_numpy_f64(case.draft_probs)
    toks = case.node_tokens.numpy()
    T = 0.9
    out = verify_tree(L, Q, toks, par, T, seed=seed + 3, offset=2)
    N = len(par)
    for b in range(60):
        acc = [True] + [None] * (N - 1)
        tight = False
        for c in range(1, N):
            u = par[c]
            p = special.softmax(L[b, u] / T)[toks[b, c]]
            ua, _ = uniforms(seed + 3, b, c, 2)
            acc[c] = ua * Q[b, u, toks[b, c]] < p
            tight |= abs(ua - p / Q[b, u, toks[b, c]]) < 1e-9
        if tight:
            continue
        best_len, best_path = -1, None
        for path in _paths(par):  # leftmost first
            n = 0
            while n + 1 < len(path) and acc[path[n + 1]]:
                n += 1
            if n > best_len:
                best_len, best_path = n, path[:n + 1]
        assert out["accept_len"][b] == best_len
        assert out["chosen"][b] == best_path[-1]
        assert list(out["path"][b, :best_len + 1]) == best_path
        assert list(out["tokens"][b, :best_len]) == [toks[b, c] for c in best_path[1:]]
        assert np.all(out["path"][b, best_len + 1:] == -1)


def test_tree_chosen_node_exact_law():
    """Tiny tree (root, 2 children, 2 grandchildren each), V = 4: enumerate all 2^6
    acceptance outcomes with their exact probabilities min(1, p/q); compare with the
    oracle's chosen-node frequencies; the bonus token follows p at the chosen node."""
    par = np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)
    V = 4
    rng = np.random.default_rng(4)
    p = rng.dirichlet(np.ones(V) * 2, size=7)
    q = rng.dirichlet(np.ones(V) * 2, size=7)
    toks = np.array([0, 1, 2, 0, 3, 1, 2], dtype=np.int32)
    B = 30000
    L = np.broadcast_to(np.log(p), (B, 7, V))
    Q = np.broadcast_to(q, (B, 7, V))
    out = verify_tree(L, Q, np.broadcast_to(toks, (B, 7)), par, 1.0, seed=11)
    a = [Fraction(1)] + [min(Fraction(1), Fraction(p[par[c], toks[c]]) / Fraction(q[par[c], toks[c]]))
                         for c in range(1, 7)]
    depth = tree_depths(par)
    law = np.zeros(7)
    for bits in itertools.product([0, 1], repeat=6):
        acc = (1,) + bits
        pr = Fraction(1)
        for c in range(1, 7):
            pr *= a[c] if acc[c] else 1 - a[c]
        alive = [True] + [False] * 6
        for c in range(1, 7):
            alive[c] = alive[par[c]] and bool(acc[c])
        best = max((c for c in range(7) if alive[c]), key=lambda c: (depth[c], -c))
        law[best] += float(pr)
    counts = np.bincount(out["chosen"], minlength=7)
    keep = law > 0
    assert counts[~keep].sum() == 0
    assert stats.chisquare(counts[keep], law[keep] * B).pvalue > 1e-3
    for c in range(7):
        sel = out["chosen"] == c
        if sel.sum() > 2000:
            d = depth[c]
            counts = np.bincount(out["tokens"][sel, d], minlength=V)
            assert stats.chisquare(counts, p[c] * sel.sum()).pvalue > 1e-3


def test_chain_tree_counts_consecutive_acceptances():
    N = 9
    par = chain_tree_parents(N)
    case = tree_case(80, par, 120, seed=7, dtype="f32", noise_sigma=0.8, sample_children=True)
    out = verify_tree(to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs),
                      case.node_tokens.numpy(), par, 1.0, seed=1)
    for b in range(80):
        acc = out["accepted"][b]
        n = 0
        while n + 1 < N and acc[n + 1]:
            n += 1
        assert out["accept_len"][b] == n
        assert list(out["path"][b, :n + 1]) == list(range(n + 1))
