"""GPU parity of the fused LM-head -> verification path (spec_lmhead_verify).

The float32 logits the MFMA GEMM writes are checked against the oracle's float64
hidden @ W within the float32-accumulation bound; verification parity is then checked
bit-exactly by running the oracle's verification on the GPU's own logits (which
separates GEMM rounding from verification decisions).
"""
import numpy as np
import pytest
import torch

import speculative_sampling_verify_03_amd as sv
from gpu_common import DEV, announce, check_linear
from oracle import lmhead_gemm_error_bound, lmhead_logits, verify_linear
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


def check_gemm_rows(got_logits, case, rows, col_block=16384):
    H = case.hidden.shape[-1]
    V = case.weight.shape[1]
    hid = to_numpy_f64(case.hidden.reshape(-1, H)[rows])
    g = got_logits.reshape(-1, V)[rows].double().numpy()
    worst = 0.0
    for c0 in range(0, V, col_block):
        w = to_numpy_f64(case.weight[:, c0:c0 + col_block])
        ref = lmhead_logits(hid, w)
        bound = lmhead_gemm_error_bound(hid, w)
        err = np.abs(g[:, c0:c0 + col_block] - ref)
        assert np.all(np.isfinite(g[:, c0:c0 + col_block]))
        assert np.all(err <= bound), f"GEMM error {err.max():.3g} above bound at columns {c0}+"
        worst = max(worst, float(err.max()))
    announce(f"GEMM rows {len(rows)}: max |err| {worst:.3g}")


def check_verify_on_gpu_logits(got, case, seed, offset=0, what=""):
    ref = verify_linear(got["logits"].double().numpy(), to_numpy_f64(case.draft_probs),
                        case.draft_tokens.numpy(), case.temperature, seed, offset)
    check_linear(got, ref, case.draft_probs.dtype, X=case.draft_tokens.numpy(), V=case.weight.shape[1],
                 what=what)


@pytest.mark.parametrize("B,k,H,V", [(2, 5, 128, 1000), (3, 2, 256, 1001), (40, 5, 64, 2048), (1, 0, 64, 64),
                                     (7, 3, 512, 4100)])
def test_lmhead_small(B, k, H, V):
    case = lmhead_case(B, k, H, V, seed=B * 100 + V)
    announce(f"lmhead B={B} k={k} H={H} V={V}")
    got = run_lmhead(case, seed=3)
    check_gemm_rows(got["logits"], case, list(range(B * (k + 1))))
    check_verify_on_gpu_logits(got, case, 3, what=f"lmhead verify B={B} k={k} V={V}")


def test_lmhead_cfg4_full():
    case = cfg4_case()
    announce("lmhead B=32 k=5 H=8192 V=128256 (generated)")
    got = run_lmhead(case, seed=0)
    rows = [0, 1, 5, 37, 100, 150, 191]
    check_gemm_rows(got["logits"], case, rows)
    check_verify_on_gpu_logits(got, case, 0, what="lmhead verify B=32 k=5 V=128256")
