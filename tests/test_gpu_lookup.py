"""GPU parity of prompt-lookup drafting (spec_lookup_drafts) against oracle/lookup.py:
bit-exact drafts and counts on histories with repeated phrases, and on the edges (empty
and one-token histories, lengths past the capacity, the largest phrase and draft
lengths)."""
import numpy as np
import pytest
import torch

import speculative_sampling_verify_03_amd as sv
from gpu_common import announce
from oracle import lookup_drafts
from synthetic import lookup_histories

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu(hist, lens, mn, mx, k):
    H = torch.as_tensor(np.asarray(hist), dtype=torch.int32, device=DEV).contiguous()
    L = torch.as_tensor(np.asarray(lens), dtype=torch.int32, device=DEV).contiguous()
    d = torch.full((H.shape[0], k), -5, dtype=torch.int32, device=DEV)
    c = torch.full((H.shape[0],), -5, dtype=torch.int32, device=DEV)
    sv.spec_lookup_drafts(H, L, mn, mx, d, c)
    torch.cuda.synchronize()
    return d.cpu().numpy(), c.cpu().numpy()


def _check(hist, lens, mn, mx, k, what):
    gd, gc = _gpu(hist, lens, mn, mx, k)
    rd, rc = lookup_drafts(hist, lens, mn, mx, k)
    assert np.array_equal(gc, rc), f"{what}: counts"
    assert np.array_equal(gd, rd), f"{what}: drafts"
    return rc


@pytest.mark.parametrize("B,cap,vocab,mn,mx,k", [(64, 4096, 32000, 1, 3, 5), (16, 2000, 50, 2, 4, 8),
                                                 (200, 300, 7, 1, 16, 64), (8, 70000, 32000, 1, 2, 1),
                                                 (32, 3000, 20, 2, 6, 10)])
def test_lookup_random(B, cap, vocab, mn, mx, k):
    announce(f"lookup B={B} cap={cap} vocab={vocab} n={mn}..{mx} k={k}")
    hist, lens = lookup_histories(B, cap, vocab=vocab, seed=B + cap)
    rc = _check(hist, lens, mn, mx, k, f"B={B} cap={cap}")
    assert (rc > 0).mean() > 0.5   # the generator repeats phrases: most sequences find one


def test_lookup_edges():
    announce("lookup edges")
    cap = 20
    hist = np.zeros((6, cap), dtype=np.int64)
    hist[0, :9] = [7, 8, 9, 1, 2, 3, 7, 8, 9]
    hist[1, :1] = [5]
    hist[3, :4] = [1, 2, 3, 4]
    hist[4, :] = np.arange(cap) % 3
    hist[5, :] = 4
    lens = np.array([9, 1, 0, 4, cap + 1, cap])   # row 4: length past the capacity
    _check(hist, lens, 1, 3, 4, "edges")
    _check(hist, lens, 3, 3, 1, "edges n=3 k=1")
    _check(hist, lens, 1, 16, 64, "edges widest")


def test_lookup_empty_batch():
    announce("lookup B=0")
    H = torch.empty((0, 10), dtype=torch.int32, device=DEV)
    L = torch.empty((0,), dtype=torch.int32, device=DEV)
    sv.spec_lookup_drafts(H, L, 1, 3, torch.empty((0, 4), dtype=torch.int32, device=DEV),
                          torch.empty((0,), dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("seed", [7, 107])
def test_lookup_bench_workload(seed):
    # the benchmark's own inputs: B=64 histories of up to 8192 tokens, phrases of 1-3, 5 drafts
    announce(f"lookup bench workload seed={seed}")
    hist, lens = lookup_histories(64, 8192, seed=seed)
    _check(hist, lens, 1, 3, 5, f"bench seed={seed}")

