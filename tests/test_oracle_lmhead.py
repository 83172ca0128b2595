"""Pins of the oracle's LM-head projection: exact rational dot products of bf16 values,
and the float32-accumulation error bound against an independent float32 matmul."""
from fractions import Fraction

import numpy as np
import torch

from oracle import lmhead_gemm_error_bound, lmhead_logits, verify_linear, verify_lmhead
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
