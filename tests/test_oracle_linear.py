"""Pins of the oracle's linear verification against what the pages and mathematics fix.

* exact rational enumeration of the whole step's law on tiny vocabularies, and the
  oracle's empirical law against it (G/chi-square);
* the emitted tokens follow the target law ("Speculative decoding explained",
  section "Draft and verification loop");
* the mean emitted length under i.i.d. acceptance alpha is (1 - alpha^{k+1}) / (1 - alpha);
* best case k+1 tokens and worst case one token per pass (same page, section "Best and
  worst case"; tests/golden/page_facts.json);
* k = 0 is plain inverse-CDF sampling (scipy's rv_discrete.ppf);
* every acceptance decision equals the exact rational comparison u * q < p;
* the acceptance probability min(1, p/q) falls as the draft grows more confident.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import (acceptance_overlap, inverse_cdf_sample, target_distribution,
                    uniforms, verify_linear)
from synthetic import fixed_pq_case, linear_case, to_numpy_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _run(case, seed=0, offset=0):
    return verify_linear(to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs),
                         case.draft_tokens.numpy(), case.temperature, seed, offset)


def _rand_dist(rng, V, zero_frac=0.0):
    # random rational distribution with denominators 64
    w = rng.integers(1, 20, size=V)
    if zero_frac:
        w[rng.random(V) < zero_frac] = 0
        if w.sum() == 0:
            w[0] = 1
    return [Fraction(int(x), int(w.sum())) for x in w]


def exact_law(p, q):
    """Exact law of the emitted tuple of one speculative step, by enumeration over the
    draft tokens and both outcomes of every acceptance test (independent of the oracle:
    it follows the probabilities, not the draws)."""
    k = len(q)
    V = len(p[0])
    law = {}

    def add(t, pr):
        law[t] = law.get(t, Fraction(0)) + pr

    def rec(j, prefix, pr):
        if j == k:
            for y in range(V):
                if p[k][y]:
                    add(prefix + (y,), pr * p[k][y])
            return
        r = [max(Fraction(0), p[j][v] - q[j][v]) for v in range(V)]
        S = sum(r)
        for x in range(V):
            if q[j][x] == 0:
                continue
            a = min(Fraction(1), p[j][x] / q[j][x])
            if a > 0:
                rec(j + 1, prefix + (x,), pr * q[j][x] * a)
            if a < 1:
                for y in range(V):
                    if r[y]:
                        add(prefix + (y,), pr * q[j][x] * (1 - a) * r[y] / S)

    rec(0, (), Fraction(1))
    return law


@pytest.mark.parametrize("V,k,seed", [(3, 2, 0), (4, 1, 1), (2, 3, 2)])
def test_exact_law_has_target_marginals(V, k, seed):
    """The enumerated law emits, at every reached position j, a token with law p_j."""
    rng = np.random.default_rng(seed)
    p = [_rand_dist(rng, V) for _ in range(k + 1)]
    q = [_rand_dist(rng, V, zero_frac=0.3) for _ in range(k)]
    law = exact_law(p, q)
    assert sum(law.values()) == 1
    for j in range(k + 1):
        reach = sum(pr for t, pr in law.items() if len(t) > j)
        for y in range(V):
            m = sum(pr for t, pr in law.items() if len(t) > j and t[j] == y)
            assert m == reach * p[j][y]


def _gtest(counts, expected):
    counts = np.asarray(counts, dtype=np.float64)
    expected = np.asarray(expected, dtype=np.float64)
    keep = expected > 0
    assert counts[~keep].sum() == 0, "oracle emitted an impossible outcome"
    return stats.chisquare(counts[keep], expected[keep] * counts.sum() / expected[keep].sum()).pvalue


@pytest.mark.parametrize("V,k,seed", [(3, 2, 10), (4, 1, 11)])
def test_oracle_matches_exact_law(V, k, seed):
    rng = np.random.default_rng(seed)
    p = [_rand_dist(rng, V) for _ in range(k + 1)]
    q = [_rand_dist(rng, V, zero_frac=0.25) for _ in range(k)]
    law = exact_law(p, q)
    B = 40000
    case = fixed_pq_case(np.array(p, dtype=np.float64), np.array(q, dtype=np.float64),
                         B, seed=seed, dtype="f32")
    out = _run(case, seed=seed)
    keys = sorted(law)
    idx = {t: i for i, t in enumerate(keys)}
    counts = np.zeros(len(keys))
    for b in range(B):
        n = out["accept_len"][b]
        t = tuple(int(v) for v in out["tokens"][b, :n + 1])
        assert t in idx, f"impossible outcome {t}"
        counts[idx[t]] += 1
    assert _gtest(counts, [float(law[t]) for t in keys]) > 1e-3


def test_chisquare_emitted_tokens_follow_target():
    """V = 8, p != q, everything positive: the token emitted at position 0 follows p_0
    and, given the step reached position j, the token emitted there follows p_j."""
    rng = np.random.default_rng(5)
    V, k = 8, 2
    p = rng.dirichlet(np.ones(V), size=k + 1)
    q = rng.dirichlet(np.ones(V), size=k)
    B = 60000
    out = _run(fixed_pq_case(p, q, B, seed=5, dtype="f32"), seed=5)
    for j in range(k + 1):
        reached = out["accept_len"] >= j
        toks = out["tokens"][reached, j]
        counts = np.bincount(toks, minlength=V)
        assert stats.chisquare(counts, p[j] * reached.sum()).pvalue > 1e-3


@pytest.mark.parametrize("alpha", [0.3, 0.6, 0.75, 0.9])
@pytest.mark.parametrize("k", [1, 4, 8])
def test_closed_form_mean_emitted(alpha, k):
    """Same (p, q) at every position with sum min(p, q) = alpha, drafts drawn from q:
    E[emitted] = (1 - alpha^(k+1)) / (1 - alpha)."""
    V = 8
    q = np.array([0.25, 0.25, 0.25, 0.25, 0, 0, 0, 0], dtype=np.float64)
    p = alpha * q
    p[7] += 1.0 - alpha
    assert abs(acceptance_overlap(p, q) - alpha) < 1e-12
    B = 3000
    out = _run(fixed_pq_case(np.tile(p, (k + 1, 1)), np.tile(q, (k, 1)), B,
                             seed=100 + k, dtype="f32"), seed=int(alpha * 100) + k)
    emitted = out["accept_len"].astype(np.float64) + 1
    expect = (1 - alpha ** (k + 1)) / (1 - alpha)
    se = emitted.std(ddof=1) / np.sqrt(B)
    assert abs(emitted.mean() - expect) < 4 * se + 1e-9
    # accepted drafts: E[n] = alpha (1 - alpha^k) / (1 - alpha)
    assert abs(out["accept_len"].mean() - alpha * (1 - alpha ** k) / (1 - alpha)) < 4 * se + 1e-9


def test_best_case_emits_k_plus_one():
    facts = json.load(open(GOLDEN))["tokens_per_pass_best_case"]["emitted_for_k"]
    for k_s, emitted in facts.items():
        k = int(k_s)
        case = linear_case(50, k, 64, seed=k, dtype="f32")
        # draft probabilities equal to the target's own distribution: nothing is rejected
        L = to_numpy_f64(case.logits)
        Q = np.stack([[target_distribution(L[b, j], 1.0) for j in range(k)] for b in range(50)])
        out = verify_linear(L, Q, case.draft_tokens.numpy(), 1.0, seed=3)
        ok = ~out["near_tie"]
        assert ok.sum() >= 45
        assert np.all(out["accept_len"][ok] + 1 == emitted)
        assert np.all(out["tokens"][ok] >= 0)


def test_worst_case_disjoint_supports_emits_one():
    facts = json.load(open(GOLDEN))["tokens_per_pass_worst_case"]
    V, k = 8, 5
    p = np.zeros((k + 1, V))
    p[:, :4] = 0.25
    q = np.zeros((k, V))
    q[:, 4:] = 0.25
    out = _run(fixed_pq_case(p, q, 2000, seed=9, dtype="f32"), seed=9)
    assert np.all(out["accept_len"] + 1 == facts["emitted"])
    assert np.all(out["tokens"][:, 0] < 4) and np.all(out["tokens"][:, 1:] == -1)
    counts = np.bincount(out["tokens"][:, 0], minlength=4)
    assert stats.chisquare(counts).pvalue > 1e-3


def test_k0_is_inverse_cdf_sampling():
    V = 16
    rng = np.random.default_rng(2)
    p = rng.dirichlet(np.ones(V) * 0.5)
    case = fixed_pq_case(p[None, :], np.zeros((0, V)), 3000, seed=1, dtype="f32")
    L = to_numpy_f64(case.logits)
    out = verify_linear(L, np.zeros((3000, 0, V)), np.zeros((3000, 0), np.int32), 1.0, seed=21)
    assert np.all(out["accept_len"] == 0)
    for b in range(3000):
        pb = target_distribution(L[b, 0], 1.0)
        _, us = uniforms(21, b, 0, 0)
        rv = stats.rv_discrete(values=(np.arange(V), pb))
        cdf = np.cumsum(pb)
        if np.min(np.abs(cdf - us)) < 1e-12:
            continue  # ppf takes CDF >= u, the sampler CDF > u: differ only on equality
        assert out["tokens"][b, 0] == int(rv.ppf(us))


def test_decisions_match_rational_comparison():
    case = linear_case(200, 6, 50, seed=4, dtype="bf16", noise_sigma=1.0)
    L = to_numpy_f64(case.logits)
    Q = to_numpy_f64(case.draft_probs)
    X = case.draft_tokens.numpy()
    out = verify_linear(L, Q, X, 1.3, seed=8, offset=5)
    for b in range(200):
        for j in range(6):
            x = int(X[b, j])
            p = special.softmax(L[b, j] / 1.3)[x]
            ua, _ = uniforms(8, b, j, 5)
            exact = Fraction(ua) * Fraction(float(Q[b, j, x])) < Fraction(float(p))
            if abs(ua - p / Q[b, j, x]) > 1e-12:
                assert out["accepted"][b, j] == exact
            assert abs(out["target_prob"][b, j] - p) < 1e-12
        n = out["accept_len"][b]
        first_rej = np.nonzero(~out["accepted"][b])[0]
        assert n == (first_rej[0] if first_rej.size else 6)
        assert np.array_equal(out["tokens"][b, :n], X[b, :n])
        assert np.all(out["tokens"][b, n + 1:] == -1)


def test_residual_draw_only_where_target_exceeds_draft():
    """A correction token always has p(y) > q(y) at the rejected row."""
    case = linear_case(300, 3, 40, seed=6, dtype="f32", noise_sigma=1.5)
    L = to_numpy_f64(case.logits)
    Q = to_numpy_f64(case.draft_probs)
    out = verify_linear(L, Q, case.draft_tokens.numpy(), 1.0, seed=6)
    rej = out["accept_len"] < 3
    assert rej.sum() > 50
    for b in np.nonzero(rej)[0]:
        n = out["accept_len"][b]
        y = out["tokens"][b, n]
        assert target_distribution(L[b, n], 1.0)[y] > Q[b, n, y]


def test_acceptance_probability_monotone_in_draft_confidence():
    V = 8
    p = np.full((2, V), 1.0 / V)
    aps = []
    for qx in np.linspace(0.05, 0.9, 12):
        q = np.full((1, V), (1 - qx) / (V - 1))
        q[0, 3] = qx
        L = np.log(p)[None]
        out = verify_linear(L, q[None], np.array([[3]]), 1.0, seed=0)
        aps.append(out["accept_prob"][0, 0])
        assert out["accept_prob"][0, 0] == pytest.approx(min(1.0, (1.0 / V) / qx), rel=1e-12)
    assert all(a >= b for a, b in zip(aps, aps[1:]))
    assert aps[0] == 1.0 and aps[-1] < 0.2


def test_out_of_range_token_is_rejected():
    case = linear_case(4, 3, 32, seed=1, dtype="f32")
    X = case.draft_tokens.numpy().copy()
    X[:, 1] = [-1, 32, 10**6, -(10**6)]
    out = verify_linear(to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs), X, 1.0, seed=0)
    assert np.all(out["accept_len"] <= 1)
    assert np.all(~out["accepted"][:, 1]) and np.all(out["target_prob"][:, 1] == 0)


def test_minus_inf_logits_have_zero_mass():
    V, k = 8, 1
    L = np.zeros((500, 2, V))
    L[:, :, 4:] = -np.inf
    Q = np.full((500, 1, V), 1.0 / V)
    X = np.tile(np.arange(V, dtype=np.int32), 63)[:500, None]
    out = verify_linear(L, Q, X, 1.0, seed=2)
    assert np.all(out["tokens"][out["tokens"] >= 0] < 4)
    assert np.all(out["accepted"][:, 0] == (X[:, 0] < 4))


def test_target_distribution_matches_scipy():
    rng = np.random.default_rng(0)
    for T in (0.3, 0.7, 1.0, 2.5):
        l = rng.normal(0, 3, size=1000)
        assert np.allclose(target_distribution(l, T), special.softmax(l / T), rtol=1e-12, atol=0)


def test_inverse_cdf_boundaries():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert inverse_cdf_sample(w, 0.0)[0] == 1
    assert inverse_cdf_sample(w, 0.25 - 2**-24)[0] == 1
    assert inverse_cdf_sample(w, 0.25)[0] == 3  # C_i > t: the boundary goes right
    assert inverse_cdf_sample(w, 0.75)[0] == 4
    assert inverse_cdf_sample(w, 1 - 2**-24)[0] == 4
    # unnormalised weights scale t with S
    assert inverse_cdf_sample(4 * w, 0.5)[0] == 3


def test_offset_changes_draws_and_is_reproducible():
    case = linear_case(64, 4, 100, seed=3, dtype="f32", noise_sigma=1.0)
    a = _run(case, seed=1, offset=0)
    b = _run(case, seed=1, offset=0)
    c = _run(case, seed=1, offset=1)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert not np.array_equal(a["tokens"], c["tokens"])


def test_seq_base_verifies_one_sequence_of_a_batch():
    """Sequence b of a batch, verified on its own with seq_base = b, gives the batch's row b."""
    case = linear_case(6, 3, 40, seed=12, dtype="f32", noise_sigma=1.0)
    L, Q, X = to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs), case.draft_tokens.numpy()
    full = verify_linear(L, Q, X, 1.0, seed=4, offset=2)
    for b in range(6):
        one = verify_linear(L[b:b + 1], Q[b:b + 1], X[b:b + 1], 1.0, seed=4, offset=2, seq_base=b)
        assert np.array_equal(one["tokens"][0], full["tokens"][b])
        assert one["accept_len"][0] == full["accept_len"][b]


def test_u_shift_moves_a_near_tie_decision():
    """The u_shift hook: with p/q set to the position's own u_acc plus 5e-7, the test
    accepts; moving u_acc up by 1e-6 rejects it.  A zero shift changes nothing."""
    from oracle import uniforms
    V = 4
    u_acc, _ = uniforms(3, 0, 0, 0)
    q = np.array([[[0.25, 0.25, 0.25, 0.25]]])
    ratio = u_acc + 5e-7
    p0 = ratio * 0.25
    rest = (1.0 - p0) / 3.0
    L = np.log(np.array([[[p0, rest, rest, rest], [0.25, 0.25, 0.25, 0.25]]]))
    X = np.array([[0]])
    base = verify_linear(L, q, X, 1.0, seed=3)
    assert base["accept_len"][0] == 1 and base["near_tie"][0]
    assert np.array_equal(verify_linear(L, q, X, 1.0, seed=3, u_shift=(0.0, 0.0))["tokens"], base["tokens"])
    up = verify_linear(L, q, X, 1.0, seed=3, u_shift=(1e-6, 0.0))
    assert up["accept_len"][0] == 0
    assert V == L.shape[-1]


def test_residual_mass_is_reported():
    """residual_mass is sum max(0, p_n - q_n) after a rejection and 1 after a full accept."""
    case = linear_case(16, 2, 30, seed=13, dtype="f32", noise_sigma=1.5)
    L, Q, X = to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs), case.draft_tokens.numpy()
    out = verify_linear(L, Q, X, 1.0, seed=1)
    for b in range(16):
        n = out["accept_len"][b]
        if n < 2 and not out["fallback"][b]:
            p = target_distribution(L[b, n], 1.0)
            assert np.isclose(out["residual_mass"][b], np.maximum(0.0, p - Q[b, n]).sum(), rtol=1e-12)
        else:
            assert out["residual_mass"][b] == 1.0
