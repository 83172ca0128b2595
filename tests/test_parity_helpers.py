"""CPU checks of the parity helpers the GPU tests rely on: how a near-tie sequence on which
a result differs from the oracle is accepted or refused."""
import numpy as np
import pytest

from gpu_common import explain_near_ties, oracle_linear_f64
from oracle import uniforms


def _tie_case():
    """One sequence, k = 1, V = 6: position 0 accepts surely; the bonus draw from p_1 has
    u_smp 2e-7 above the start of token 4, with token 3 (mass 1e-7) just before it, so the
    draw moved by -1e-6 lands on token 2 and by +1e-6 stays on token 4."""
    _, u = uniforms(1, 0, 1, 0)
    p1 = np.full(6, 1e-3)
    p1[3] = 1e-7
    head = u - 0.3e-6 - 2e-3     # C_2 = u - 0.3e-6 (normalised, mass 1 in total)
    p1[0] = head
    p1[1:3] = 1e-3
    p1[4] = 1e-3
    p1[5] = 1.0 - p1[:5].sum()
    L = np.log(np.stack([np.array([0.9, 0.02, 0.02, 0.02, 0.02, 0.02]), p1]))[None]
    Q = np.array([[[0.5, 0.1, 0.1, 0.1, 0.1, 0.1]]])
    X = np.array([[0]])
    ref = oracle_linear_f64(L, Q, X, 1.0, 1)
    assert ref["near_tie"][0] and ref["accept_len"][0] == 1
    return ref


def _got(ref, token):
    t = ref["tokens"].copy()
    t[0, 1] = token
    return dict(tokens=t, accept_len=ref["accept_len"].copy())


def test_draw_between_shifted_outcomes_is_explained():
    ref = _tie_case()
    y0 = int(ref["tokens"][0, 1])
    assert y0 == 4
    for tok in (2, 3, 4):  # token 3 (mass 1e-7) lies inside the sweep without being hit by its ends
        got = _got(ref, tok)
        diff = np.array([tok != y0])
        assert explain_near_ties(got, ref, diff, "helper") == int(diff[0])


@pytest.mark.parametrize("tok", [1, 5])
def test_draw_outside_the_sweep_is_refused(tok):
    ref = _tie_case()
    got = _got(ref, tok)
    with pytest.raises(AssertionError, match="outside what draws within 1e-6"):
        explain_near_ties(got, ref, np.array([True]), "helper")


def test_wrong_length_is_refused():
    ref = _tie_case()
    got = dict(tokens=np.array([[4, -1]]), accept_len=np.array([0]))
    with pytest.raises(AssertionError, match="outside what draws within 1e-6"):
        explain_near_ties(got, ref, np.array([True]), "helper")
