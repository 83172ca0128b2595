"""GPU parity of the fused LM-head -> verification path (spec_lmhead_verify).

Three checks per case:
  * the float32 logits the MFMA GEMM writes, every row, against the oracle's float64
    hidden @ W: inside the worst-case fp32-accumulation bound and inside the much tighter
    probabilistic bound (oracle.lmhead_gemm_error_bound_probabilistic, which one left-out
    product already exceeds);
  * verification bit-exact against the oracle run on the GPU's own logits (separates the
    GEMM's rounding from the verification decisions);
  * verification against the oracle run from the inputs (hidden @ W in float64): bit-exact
    except sequences whose deciding draw lies within what the GEMM's measured logit error
    could move (a logit error of at most eps changes every p by a factor within
    exp(+-2 eps / T), so a threshold p/q moves by at most 2 delta and a normalised CDF
    value by at most 2 delta / (S - delta), delta = exp(2 eps / T) - 1, S the draw's mass);
    those are counted as near-ties.
"""
import numpy as np
import pytest
import torch

import speculative_sampling_verify_03_amd as sv
import tie_report
from gpu_common import DEV, NEAR, announce, check_linear, oracle_linear_f64
from oracle import lmhead_gemm_error_bound, lmhead_gemm_error_bound_probabilistic, lmhead_logits
from synthetic import cfg4_case, lmhead_case, to_numpy_f64

pytestmark = pytest.mark.gpu


def run_lmhead(case, seed, offset=0):
    B, R, H = case.hidden.shape
    k = R - 1
    V = case.weight.shape[1]
    h = case.hidden.to(DEV)
    w = case.weight.to(DEV)
    q = case.draft_probs.to(DEV)
    x = case.draft_tokens.to(DEV)
    logits = torch.full((B, R, V), float("nan"), dtype=torch.float32, device=DEV)
    toks = torch.full((B, R), -7, dtype=torch.int32, device=DEV)
    alen = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    tp = torch.empty((B, k), dtype=torch.float32, device=DEV)
    ap = torch.empty((B, k), dtype=torch.float32, device=DEV)
    ws = sv.new_workspace(sv.SV_KIND_LMHEAD, B, k, V, H)
    sv.spec_lmhead_verify(h, w, q, x, case.temperature, seed, offset, logits, toks, alen, tp, ap, ws)
    torch.cuda.synchronize()
    return dict(logits=logits.cpu(), tokens=toks.cpu().numpy(), accept_len=alen.cpu().numpy(),
                target_prob=tp.cpu().numpy(), accept_prob=ap.cpu().numpy())


def check_gemm(got_logits, case, what, col_block=8192):
    """Every row of the GEMM's output against float64 hidden @ W, within both bounds.
    Returns the exact logits [M, V]."""
    H = case.hidden.shape[-1]
    V = case.weight.shape[1]
    hid = to_numpy_f64(case.hidden.reshape(-1, H))
    g = got_logits.reshape(-1, V).double().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite logits"
    exact = np.empty_like(g)
    max_err = max_ratio = 0.0
    sq_err = sq_ref = 0.0
    for c0 in range(0, V, col_block):
        c1 = min(V, c0 + col_block)
        w = to_numpy_f64(case.weight[:, c0:c1])
        ref = lmhead_logits(hid, w)
        exact[:, c0:c1] = ref
        err = np.abs(g[:, c0:c1] - ref)
        worst = lmhead_gemm_error_bound(hid, w)
        tight = lmhead_gemm_error_bound_probabilistic(hid, w)
        assert np.all(err <= worst), f"{what}: GEMM error {err.max():.3g} above the worst-case bound at {c0}+"
        over = err > tight
        assert not over.any(), (f"{what}: GEMM error above the probabilistic bound at "
                                f"{np.argwhere(over)[:3] + [0, c0]}: {err[over][:3]} > {tight[over][:3]}")
        max_err = max(max_err, float(err.max()))
        max_ratio = max(max_ratio, float((err / tight).max()))
        sq_err += float((err ** 2).sum())
        sq_ref += float((ref ** 2).sum())
    line = (f"{what}: GEMM {g.shape[0]} rows x {V}: max |err| {max_err:.3g}, max |err| / probabilistic bound "
            f"{max_ratio:.3g}, relative RMS error {np.sqrt(sq_err / max(sq_ref, 1e-300)):.3g}")
    announce(line)
    tie_report.add(line)
    return exact


def check_verify_on_gpu_logits(got, case, seed, offset=0, what=""):
    ref = oracle_linear_f64(got["logits"].double().numpy(), to_numpy_f64(case.draft_probs),
                            case.draft_tokens.numpy(), case.temperature, seed, offset)
    check_linear(got, ref, case.draft_probs.dtype, X=case.draft_tokens.numpy(), V=case.weight.shape[1],
                 what=what)


def check_verify_from_inputs(got, case, exact, seed, offset=0, what=""):
    B, R, _ = case.hidden.shape
    V = case.weight.shape[1]
    T = case.temperature
    ref = oracle_linear_f64(exact.reshape(B, R, V), to_numpy_f64(case.draft_probs), case.draft_tokens.numpy(), T,
                            seed, offset)
    eps = np.abs(got["logits"].double().numpy().reshape(B, R, V) - exact.reshape(B, R, V)).max(axis=(1, 2))
    delta = np.expm1(2.0 * eps / T)
    S = ref["residual_mass"]
    gemm_tie = ((ref["acc_margin"] < NEAR + 2.0 * delta)
                | (ref["smp_margin"] < NEAR + 2.0 * delta / np.maximum(S - delta, 1e-300)))
    ok = ~(ref["near_tie"] | gemm_tie)
    diff = (got["accept_len"] != ref["accept_len"]) | np.any(got["tokens"] != ref["tokens"], axis=1)
    bad = np.nonzero(ok & diff)[0]
    assert bad.size == 0, (f"{what}: {bad.size} sequences differ from the oracle run from the inputs, first "
                           f"{bad[:3]}: gpu {got['tokens'][bad[:2]]} / oracle {ref['tokens'][bad[:2]]}")
    line = (f"{what} (oracle from hidden @ W): {int(ok.sum())} of {B} bit-exact; {int((~ok).sum())} within the "
            f"GEMM's reach or a 1e-6 near-tie ({int((~ok & ~diff).sum())} match anyway); max logit error "
            f"{eps.max():.3g}")
    announce(line)
    tie_report.add(line)


# M = B * (k + 1) rows; V % 8 == 0 with aligned rows takes the direct-to-LDS kernel (16-row
# blocks: up to 4, 8 or 12 per workgroup), other V the register-prefetch kernel (8-byte W
# loads when V % 4 == 0, element loads otherwise).
@pytest.mark.parametrize("B,k,H,V", [
    (2, 5, 128, 1000), (3, 2, 256, 1001), (40, 5, 64, 2048), (1, 0, 64, 64), (7, 3, 512, 4100),
    (16, 5, 256, 4096),   # M = 96: direct kernel, 8 blocks
    (13, 4, 128, 3000),   # M = 65: direct kernel, 8 blocks, one row in the last block
    (32, 3, 64, 2048),    # M = 128: direct kernel, 8 full blocks
    (20, 3, 128, 2004),   # M = 80: 8-byte fallback, 8 blocks
    (32, 3, 64, 1003),    # M = 128: element fallback, 8 blocks
    (25, 5, 128, 2006),   # M = 150: element fallback, 12 blocks
    (30, 6, 64, 1012),    # M = 210: 8-byte fallback, 12 blocks, two block rows
])
def test_lmhead_small(B, k, H, V):
    case = lmhead_case(B, k, H, V, seed=B * 100 + V)
    what = f"lmhead B={B} k={k} H={H} V={V}"
    announce(what)
    got = run_lmhead(case, seed=3)
    exact = check_gemm(got["logits"], case, what)
    check_verify_on_gpu_logits(got, case, 3, what=what)
    check_verify_from_inputs(got, case, exact, 3, what=what)


def test_lmhead_cfg4_full():
    case = cfg4_case()
    what = "lmhead B=32 k=5 H=8192 V=128256"
    announce(what + " (generated)")
    got = run_lmhead(case, seed=0)
    exact = check_gemm(got["logits"], case, what)
    check_verify_on_gpu_logits(got, case, 0, what=what)
    check_verify_from_inputs(got, case, exact, 0, what=what)


# The direct kernel (V % 8 == 0, aligned W and logits) also writes per-block softmax
# partials, and verification then runs from them (decide, then a chunked draw); the cases
# below pin that path at its edges.
@pytest.mark.parametrize("B,k,H,V,T,qt", [(24, 4, 128, 20000, 0.7, torch.bfloat16),
                                          (9, 7, 64, 33000, 1.5, torch.float32),
                                          (64, 1, 64, 8200, 1.0, torch.bfloat16)])
def test_lmhead_fused_shapes(B, k, H, V, T, qt):
    case = lmhead_case(B, k, H, V, seed=B + V, temperature=T)
    case.draft_probs = case.draft_probs.to(qt)
    what = f"lmhead fused B={B} k={k} H={H} V={V} T={T} q={qt}"
    announce(what)
    got = run_lmhead(case, seed=7, offset=3)
    exact = check_gemm(got["logits"], case, what)
    check_verify_on_gpu_logits(got, case, 7, offset=3, what=what)
    check_verify_from_inputs(got, case, exact, 7, offset=3, what=what)


def test_lmhead_fused_invalid_tokens():
    # out-of-range draft tokens are rejected (p(x) = 0), so those sequences draw their
    # residual at that position
    B, k, H, V = 16, 3, 64, 4096
    case = lmhead_case(B, k, H, V, seed=5)
    case.draft_tokens[:, 1] = torch.tensor([-1, V, 10**6, -(10**6)] * 4, dtype=torch.int32)
    got = run_lmhead(case, seed=2)
    check_verify_on_gpu_logits(got, case, 2, what="lmhead fused invalid tokens")
    assert np.all(got["accept_len"] <= 1)


def test_lmhead_fused_empty_residual():
    # hidden = e_0, W row 0 = 1000 at one column and 0 elsewhere: every row's p is one-hot
    # (the other terms, e^-1000, underflow to zero in float32 and in float64 alike), q is the
    # same one-hot and the draft token is another column (q(x) = p(x) = 0): rejected,
    # max(0, p - q) = 0 everywhere, and the token is drawn from p itself: the hot column
    B, k, H, V, hot = 8, 2, 64, 2048, 1234
    hidden = torch.zeros((B, k + 1, H), dtype=torch.bfloat16)
    hidden[:, :, 0] = 1.0
    w = torch.zeros((H, V), dtype=torch.bfloat16)
    w[0, hot] = 1000.0
    q = torch.zeros((B, k, V), dtype=torch.float32)
    q[:, :, hot] = 1.0
    from synthetic.generators import LMHeadCase
    case = LMHeadCase(hidden=hidden, weight=w, draft_probs=q,
                      draft_tokens=torch.full((B, k), 7, dtype=torch.int32), temperature=1.0, meta={})
    got = run_lmhead(case, seed=1)
    check_verify_on_gpu_logits(got, case, 1, what="lmhead fused empty residual")
    assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] == hot)


@pytest.mark.parametrize("B,k,H,V", [(4, 3, 128, 1000), (16, 5, 256, 4096), (32, 5, 8192, 128256)])
def test_lmhead_logits_alone(B, k, H, V):
    # spec_lmhead_logits: the same kernels (and bits) as the logits spec_lmhead_verify writes
    case = cfg4_case() if V == 128256 else lmhead_case(B, k, H, V, seed=B * 7 + V)
    what = f"lmhead logits alone M={B * (k + 1)} H={H} V={V}"
    announce(what)
    got = run_lmhead(case, seed=3)
    alone = torch.full((B, k + 1, V), float("nan"), dtype=torch.float32, device=DEV)
    sv.spec_lmhead_logits(case.hidden.to(DEV), case.weight.to(DEV), alone)
    torch.cuda.synchronize()
    assert torch.equal(alone.cpu(), got["logits"]), f"{what}: logits differ from the verify call's"
    if V != 128256:
        check_gemm(alone.cpu(), case, what)
