"""Pins of the oracle's LM-head projection: exact rational dot products of bf16 values,
and the float32-accumulation error bound against an independent float32 matmul."""
from fractions import Fraction

import numpy as np
import torch

from oracle import (lmhead_gemm_error_bound, lmhead_gemm_error_bound_probabilistic, lmhead_logits, verify_linear,
                    verify_lmhead)
from synthetic import lmhead_case, to_numpy_f64


def test_lmhead_logits_exact_on_small_case():
    case = lmhead_case(2, 2, 64, 40, seed=1)
    h = to_numpy_f64(case.hidden).reshape(-1, 64)
    w = to_numpy_f64(case.weight)
    got = lmhead_logits(h, w)
    for m in range(h.shape[0]):
        for v in range(0, 40, 7):
            exact = sum(Fraction(float(h[m, i])) * Fraction(float(w[i, v])) for i in range(64))
            assert abs(Fraction(float(got[m, v])) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**80)


def test_fp32_matmul_within_bound():
    case = lmhead_case(3, 3, 1024, 300, seed=2)
    h = case.hidden.reshape(-1, 1024)
    ref = lmhead_logits(to_numpy_f64(h), to_numpy_f64(case.weight))
    bound = lmhead_gemm_error_bound(to_numpy_f64(h), to_numpy_f64(case.weight))
    f32 = (h.to(torch.float32) @ case.weight.to(torch.float32)).double().numpy()
    assert np.all(np.abs(f32 - ref) <= bound)
    assert np.abs(f32 - ref).max() < 0.05 * bound.max()  # typical error is far inside the worst case


def test_verify_lmhead_is_projection_then_linear():
    case = lmhead_case(4, 3, 128, 96, seed=3)
    h = to_numpy_f64(case.hidden)
    w = to_numpy_f64(case.weight)
    Q = to_numpy_f64(case.draft_probs)
    X = case.draft_tokens.numpy()
    a = verify_lmhead(h, w, Q, X, 1.0, seed=5)
    b = verify_linear(h @ w, Q, X, 1.0, seed=5)
    assert np.array_equal(a["tokens"], b["tokens"])


def _k8192_case():
    """Rows of the B=32, k=5, H=8192 workload's statistics (hidden ~ N(0, 1), W ~ N(0, 0.02^2),
    both bf16) over 4096 columns: 12 rows x K = 8192."""
    case = lmhead_case(2, 5, 8192, 4096, seed=9)
    h = case.hidden.reshape(-1, 8192)
    return h, case.weight, to_numpy_f64(h), to_numpy_f64(case.weight)


def test_probabilistic_bound_holds_for_fp32_matmul():
    """An independent float32 matmul (torch's CPU GEMM, fp32 accumulation) of the bf16
    values stays inside the probabilistic bound, and the bound sits well inside the
    worst-case one at K = 8192."""
    h, w, hd, wd = _k8192_case()
    ref = lmhead_logits(hd, wd)
    tight = lmhead_gemm_error_bound_probabilistic(hd, wd)
    worst = lmhead_gemm_error_bound(hd, wd)
    err = np.abs((h.float() @ w.float()).double().numpy() - ref)
    assert np.all(err <= tight)
    assert np.all(tight < worst / 10)
    # the bound is loose on random data (errors cancel), but not by orders of magnitude
    # more than the worst-case analysis already is
    assert err.max() > 1e-5 * tight.max()


def test_dropped_product_fails_tight_bound_but_passes_worst_case():
    """A planted mistake the worst-case bound cannot see: one k-row of the contraction left
    out (hidden[:, h] = 0 for the h whose largest |hidden| is smallest, so every error
    a_h * w_hv is small).  The worst-case bound still passes everywhere; the probabilistic
    bound fails on a large share of the entries."""
    h, w, hd, wd = _k8192_case()
    ref = lmhead_logits(hd, wd)
    j = int(np.argmin(np.abs(hd).max(axis=0)))
    planted = h.float().clone()
    planted[:, j] = 0.0
    err = np.abs((planted @ w.float()).double().numpy() - ref)
    assert np.all(err <= lmhead_gemm_error_bound(hd, wd))
    over = err > lmhead_gemm_error_bound_probabilistic(hd, wd)
    assert over.mean() > 0.2, over.mean()
    big = np.abs(hd[:, j]) > 0.1  # rows where the left-out product is not negligible
    assert over[big].any(axis=1).all()


def test_probabilistic_bound_formula_small_k():
    """At K = 1 there is no addition: the bound must still be positive and tiny; at K = 64
    it equals exp(10 * 8 * 2^-24 + 64 * 2^-48 / (1 - 2^-24)) - 1 times sum |a w|."""
    a = np.array([[1.5, -2.0]])
    w = np.array([[0.25], [0.5]])
    b = lmhead_gemm_error_bound_probabilistic(a, w)
    u = 2.0 ** -24
    assert np.isclose(b[0, 0], np.expm1(10 * np.sqrt(2) * u + 2 * u * u / (1 - u)) * (1.5 * 0.25 + 2.0 * 0.5))
    a64 = np.ones((1, 64))
    w64 = np.full((64, 1), 0.5)
    b64 = lmhead_gemm_error_bound_probabilistic(a64, w64)
    assert np.isclose(b64[0, 0], np.expm1(80 * u + 64 * u * u / (1 - u)) * 32.0, rtol=1e-12)
