"""GPU parity of greedy verification and static-tree verification against the oracle."""
import numpy as np
import pytest
import torch

from gpu_common import announce, check_greedy, check_tree, run_greedy, run_tree
from synthetic import (cfg3_case, cfg5_case, chain_tree_parents, eagle_tree_parents, linear_case,
                       to_numpy_f64, tree_case)

pytestmark = pytest.mark.gpu


def test_cfg3_greedy_full():
    case = cfg3_case()
    announce("greedy B=256 k=8 V=128256 bf16")
    got = run_greedy(case.logits, case.greedy_tokens)
    ref = check_greedy(got, case.logits, case.greedy_tokens, what="greedy B=256 k=8 V=128256")
    announce(f"greedy mean emitted {ref['accept_len'].mean() + 1:.3f}")


@pytest.mark.parametrize("k", [1, 4, 8])
def test_greedy_identity(k):
    case = linear_case(64, k, 32000, seed=k, dtype="bf16")
    X = torch.from_numpy(np.argmax(to_numpy_f64(case.logits)[:, :k], axis=-1).astype(np.int32))
    got = run_greedy(case.logits, X)
    assert np.all(got["accept_len"] == k)
    check_greedy(got, case.logits, X, what=f"greedy identity k={k}")


@pytest.mark.parametrize("dtype,V,misalign", [("bf16", 1001, 0), ("f32", 777, 1), ("bf16", 50257, 3),
                                              ("f32", 131072, 0), ("bf16", 5, 0)])
def test_greedy_ragged(dtype, V, misalign):
    case = linear_case(40, 5, V, seed=V, dtype=dtype, noise_sigma=0.05)
    got = run_greedy(case.logits, case.greedy_tokens, misalign)
    check_greedy(got, case.logits, case.greedy_tokens, what=f"greedy V={V} {dtype} misalign={misalign}")


def test_greedy_ties_across_splits():
    # V = 65536 with 32 rows: each row is split over 4 workgroups; equal maxima sit in
    # different splits and the lowest index must win the cross-workgroup merge
    V = 65536
    L = torch.zeros((8, 4, V), dtype=torch.bfloat16)
    L[:, :, [20000, 17, 40000, 65535]] = 3.0
    X = torch.tensor([[17, 17, 17], [20000, 17, 17], [17, 40000, 17], [17, 17, 65535]] * 2, dtype=torch.int32)
    got = run_greedy(L, X)
    assert list(got["accept_len"][:4]) == [3, 0, 1, 2]
    assert np.all(got["tokens"][:, 0] == 17)
    check_greedy(got, L, X, what="greedy ties across splits")


def test_greedy_ties_lowest_index():
    V = 4096
    L = torch.zeros((8, 4, V), dtype=torch.bfloat16)
    L[:, :, [17, 900, 2500, 4095]] = 3.0
    X = torch.tensor([[17, 17, 17], [900, 17, 17], [17, 2500, 17], [17, 17, 4095]] * 2, dtype=torch.int32)
    got = run_greedy(L, X)
    assert list(got["accept_len"][:4]) == [3, 0, 1, 2]
    assert np.all(got["tokens"][:, 0] == 17)
    check_greedy(got, L, X, what="greedy ties")


@pytest.mark.parametrize("case_seed", [5, 105, 205, 305])
def test_cfg5_tree_full(case_seed):
    # four generated batches of the page's tree: 64 sequences at full size
    announce(f"tree B=16 N=61 V=128256 bf16, inputs seed {case_seed} (generating)")
    case = cfg5_case(seed=case_seed)
    got = run_tree(case, seed=0)
    ref = check_tree(got, case, seed=0, what=f"tree B=16 N=61 V=128256 inputs {case_seed}")
    announce(f"tree mean accept_len {ref['accept_len'].mean():.3f}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("misalign", [0, 1])
def test_greedy_signed_zero_maximum(dtype, misalign):
    """Rows whose maximum is zero, held as -0.0 in one piece of the row and +0.0 in a
    later one (rows of 128256 are cut into several workgroups' pieces on both the flat
    path, misalign 0, and the split path, misalign 1).  The two compare equal, so the
    lower index wins whichever sign it carries."""
    V = 128256
    L = torch.full((2, 3, V), -1.0, dtype=dtype)
    L[0, 0, 5] = -0.0
    L[0, 0, 100000] = 0.0     # later piece, +0.0
    L[0, 1, 9] = 0.0
    L[0, 1, 90000] = -0.0     # later piece, -0.0
    L[0, 2, 64000] = -0.0
    L[0, 2, 127999] = 0.0
    L[1, :, 70000] = -0.0
    L[1, :, 120000] = 0.0
    X = torch.tensor([[5, 9], [70000, 120000]], dtype=torch.int32)
    assert int(L[0, 0, 5].view(torch.int16 if dtype == torch.bfloat16 else torch.int32)) < 0  # really -0.0
    got = run_greedy(L, X, misalign)
    assert list(got["accept_len"]) == [2, 1]
    assert list(got["tokens"][0]) == [5, 9, 64000] and list(got["tokens"][1]) == [70000, 70000, -1]
    check_greedy(got, L, X, what=f"greedy signed zero {dtype} misalign={misalign}")


@pytest.mark.parametrize("name", ["chain", "single", "wide", "deep64"])
def test_tree_shapes(name):
    if name == "chain":
        par = chain_tree_parents(9)
    elif name == "single":
        par = np.array([-1], dtype=np.int32)
    elif name == "wide":
        par = eagle_tree_parents((63,), 64)
    else:
        par = eagle_tree_parents((2, 2, 2, 2, 2, 2), 64)
    case = tree_case(48, par, 3000, seed=len(par), dtype="f32", noise_sigma=0.6, sample_children=True)
    got = run_tree(case, seed=3, offset=2)
    check_tree(got, case, seed=3, offset=2, what=f"tree {name} N={len(par)}")


@pytest.mark.parametrize("misalign", [(1, 0), (0, 3)])
def test_tree_ragged_misaligned(misalign):
    case = tree_case(20, eagle_tree_parents((3, 2, 2), 64), 1003, seed=4, dtype="bf16", noise_sigma=0.8)
    got = run_tree(case, seed=5, misalign=misalign)
    check_tree(got, case, seed=5, what=f"tree V=1003 misalign={misalign}")


@pytest.mark.parametrize("B,k,V,dtype", [(3, 4, 31992, "bf16"), (1, 0, 8, "bf16"), (7, 3, 4100, "f32"),
                                         (100, 2, 1024, "bf16")])
def test_greedy_flat_pieces_cross_rows(B, k, V, dtype):
    # rows of whole 16-byte vectors take the flat path: equal ranges of the whole tensor
    # whose boundaries fall inside rows, and rows shorter than one range
    case = linear_case(B, k, V, seed=B + V, dtype=dtype, noise_sigma=0.05)
    got = run_greedy(case.logits, case.greedy_tokens)
    check_greedy(got, case.logits, case.greedy_tokens, what=f"greedy flat B={B} k={k} V={V} {dtype}")


@pytest.mark.parametrize("misalign", [0, 1, 5])
def test_greedy_edge_vector_ties(misalign):
    # rows that are not whole 16-byte vectors take the split path, whose first and last
    # vectors are partial and merged element by element: equal maxima there and in a whole
    # vector must still resolve to the lowest index
    V = 1001
    L = torch.zeros((4, 4, V), dtype=torch.bfloat16)
    L[0, :, [0, 999]] = 3.0      # first element vs a later whole-vector element
    L[1, :, [1000]] = 3.0        # only the last element
    L[2, :, [3, 1000]] = 3.0     # an early element vs the last
    L[3, :, :] = -1.0
    L[3, :, [1000, 7]] = -0.5
    X = torch.tensor([[0, 0, 0], [1000, 1000, 0], [3, 3, 3], [7, 7, 1000]], dtype=torch.int32)
    got = run_greedy(L, X, misalign)
    assert list(got["accept_len"]) == [3, 2, 3, 2]
    check_greedy(got, L, X, what=f"greedy edge ties misalign={misalign}")


@pytest.mark.parametrize("dtype,B,k,V", [("bf16", 260, 8, 40000), ("f32", 120, 8, 40000), ("bf16", 700, 2, 40000)])
def test_greedy_flat_two_launches(dtype, B, k, V):
    """Large aligned tensors run the flat path in two launches: the first two positions of
    every sequence, then the later positions of the sequences that kept both.  Ties at
    equal maxima, signed zeros, random rows and accept lengths from 0 to k; two calls on
    one workspace, which must come back clear."""
    from gpu_common import sections_clear, status_word
    import speculative_sampling_verify_03_amd as sv
    R = k + 1
    rng = np.random.default_rng(B + k + V)
    L = np.full((B, R, V), -1.0, dtype=np.float32)
    kinds = rng.integers(0, 3, size=(B, R))
    for b in range(B):
        for j in range(R):
            if kinds[b, j] == 0:
                L[b, j] = rng.normal(size=V).astype(np.float32)
            elif kinds[b, j] == 1:
                L[b, j, rng.choice(V, size=3, replace=False)] = 3.0
            else:
                i1, i2 = sorted(rng.choice(V, size=2, replace=False))
                L[b, j, i1] = -0.0
                L[b, j, i2] = 0.0
    Lt = torch.from_numpy(L).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    g = np.argmax(Lt.float().numpy(), axis=-1)
    keep = rng.random((B, k)) < 0.8
    X = torch.from_numpy(np.where(keep, g[:, :k], (g[:, :k] + 1) % V).astype(np.int32))
    lg = Lt.to("cuda")
    ws = sv.new_workspace(sv.SV_KIND_GREEDY, B, k, V)
    for call in range(2):
        announce(f"greedy flat, two launches: B={B} k={k} V={V} {dtype} call {call}")
        out = dict(tokens=torch.full((B, R), -7, dtype=torch.int32, device="cuda"),
                   accept_len=torch.full((B,), -7, dtype=torch.int32, device="cuda"))
        sv.spec_verify_greedy(lg, X.to("cuda"), out["tokens"], out["accept_len"], ws)
        torch.cuda.synchronize()
        got = {n: t.cpu().numpy() for n, t in out.items()}
        ref = check_greedy(got, Lt, X, what=f"greedy two launches B={B} k={k} V={V} {dtype} call {call}")
        assert status_word(ws) == 0
        assert sections_clear(ws, sv.SV_KIND_GREEDY, k, V), f"call {call}: workspace not cleared"
    assert (ref["accept_len"] < 2).sum() > 0 and (ref["accept_len"] >= 2).sum() > 0
