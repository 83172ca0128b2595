"""GPU parity of linear speculative sampling (spec_verify_linear) against the oracle, at
the workload sizes and on edge cases; plus statistical tests of the kernel's output law."""
import numpy as np
import pytest
import torch
from scipy import stats

from gpu_common import announce, check_linear, oracle_linear, run_linear, sections_clear, status_word
from oracle import verify_linear
from synthetic import cfg1_case, cfg2_case, cfg3_case, fixed_pq_case, linear_case, mtp_case, to_numpy_f64

pytestmark = pytest.mark.gpu


def _case_run(case, seed=0, offset=0, misalign=(0, 0), what="", with_probs=True):
    announce(f"{what}: B={case.B} k={case.k} V={case.V} {case.logits.dtype} T={case.temperature} "
             f"misalign={misalign} probabilities={'on' if with_probs else 'off'}")
    got = run_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset,
                     misalign, with_probs=with_probs)
    ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, case.temperature, seed, offset)
    check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=case.V, what=what)
    return got, ref


def test_cfg1_batched_1000():
    _case_run(cfg1_case(B=1000), seed=0, what="B=1000 k=4 V=1024 f32")


def test_cfg1_sequential_steps():
    """The B=1, k=4, V=1024 float32 workload as stated: 1000 independent verify calls of
    one sequence, Philox seed 0, step s drawing with offset s, one workspace reused."""
    import speculative_sampling_verify_03_amd as sv
    steps = 1000
    case = cfg1_case(B=steps)
    announce(f"B=1 k=4 V=1024 f32: {steps} sequential calls")
    lg, q, x = case.logits.to("cuda"), case.draft_probs.to("cuda"), case.draft_tokens.to("cuda")
    toks = torch.full((steps, 5), -7, dtype=torch.int32, device="cuda")
    alen = torch.full((steps,), -7, dtype=torch.int32, device="cuda")
    tp = torch.full((steps, 4), -7.0, dtype=torch.float32, device="cuda")
    ap = torch.full((steps, 4), -7.0, dtype=torch.float32, device="cuda")
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, 1, 4, 1024)
    for s in range(steps):
        sv.spec_verify_linear(lg[s:s + 1], q[s:s + 1], x[s:s + 1], 1.0, 0, s, toks[s:s + 1], alen[s:s + 1],
                              tp[s:s + 1], ap[s:s + 1], ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    got = dict(tokens=toks.cpu().numpy(), accept_len=alen.cpu().numpy(), target_prob=tp.cpu().numpy(),
               accept_prob=ap.cpu().numpy())
    L, Q, X = to_numpy_f64(case.logits), to_numpy_f64(case.draft_probs), case.draft_tokens.numpy()
    refs = [verify_linear(L[s:s + 1], Q[s:s + 1], X[s:s + 1], 1.0, 0, s) for s in range(steps)]
    ref = {key: np.concatenate([r[key] for r in refs]) for key in refs[0]}
    ref["rerun"] = lambda s, sh: verify_linear(L[s:s + 1], Q[s:s + 1], X[s:s + 1], 1.0, 0, int(s), u_shift=sh)
    check_linear(got, ref, torch.float32, X=X, V=1024, what=f"B=1 k=4 V=1024 f32, {steps} sequential steps")
    announce(f"sequential steps: mean emitted {ref['accept_len'].mean() + 1:.3f}")


def test_cfg2_full():
    got, ref = _case_run(cfg2_case(), seed=0, what="B=64 k=5 V=32000 bf16")
    acc = ref["accepted"].mean()
    announce(f"B=64 k=5 V=32000: mean acceptance {acc:.3f}, mean emitted {ref['accept_len'].mean() + 1:.3f}")


def test_cfg3_full_stochastic():
    got, ref = _case_run(cfg3_case(), seed=0, what="B=256 k=8 V=128256 bf16 T=0.7")


def test_mtp_single_token_regime():
    # one drafted token per sequence, 256 sequences, Llama-3 vocabulary
    _case_run(mtp_case(), seed=0, what="B=256 k=1 V=128256 bf16 (MTP regime)")


@pytest.mark.parametrize("name,seed", [("cfg3", 1), ("mtp", 0), ("mtp", 1)])
def test_tokens_only_full_size(name, seed):
    # without p_j(x_j) outputs the rows after a sequence's first rejection stop streaming
    # once they see it; tokens and lengths must not change
    case = cfg3_case() if name == "cfg3" else mtp_case()
    _case_run(case, seed=seed, what=f"{name} tokens only, seed {seed}", with_probs=False)


@pytest.mark.parametrize("dtype,V", [("f32", 1003), ("bf16", 1001), ("f32", 5), ("bf16", 1), ("bf16", 777),
                                     ("bf16", 20001), ("f32", 10001), ("bf16", 32761),
                                     ("f32", 65537), ("bf16", 131075), ("f32", 150000), ("bf16", 200003)])
def test_ragged_and_multi_tile_vocab(dtype, V):
    B = 24 if V > 100000 else 64
    _case_run(linear_case(B, 3, V, seed=V, dtype=dtype, noise_sigma=1.0), seed=1,
              what=f"ragged V={V} {dtype}")


@pytest.mark.parametrize("dtype,V", [("bf16", 40001), ("f32", 20001), ("bf16", 65537)])
def test_many_rows_multi_tile(dtype, V):
    # 512 rows: long rows are walked in 256-thread tiles instead of 512-thread ones
    _case_run(linear_case(128, 3, V, seed=V + 7, dtype=dtype, noise_sigma=1.0), seed=6,
              what=f"many rows V={V} {dtype}")


@pytest.mark.parametrize("misalign", [(1, 0), (0, 1), (3, 5), (1, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_bases(dtype, misalign):
    _case_run(linear_case(32, 4, 5000, seed=3, dtype=dtype, noise_sigma=1.0), seed=2, misalign=misalign,
              what=f"misaligned {misalign} {dtype}")


@pytest.mark.parametrize("k", [0, 1, 63])
def test_k_extremes(k):
    _case_run(linear_case(40, k, 300, seed=k, dtype="bf16", noise_sigma=0.7), seed=4, what=f"k={k}")


@pytest.mark.parametrize("T", [0.3, 0.7, 2.5])
def test_temperatures(T):
    _case_run(linear_case(48, 5, 4000, seed=9, dtype="bf16", noise_sigma=0.5, temperature=T), seed=5,
              what=f"T={T}")


@pytest.mark.parametrize("lt,qt", [(torch.float32, torch.bfloat16), (torch.bfloat16, torch.float32)])
def test_mixed_dtypes(lt, qt):
    case = linear_case(32, 5, 9000, seed=12, dtype="f32", noise_sigma=1.0)
    case.logits = case.logits.to(lt)
    case.draft_probs = case.draft_probs.to(qt)
    _case_run(case, seed=6, what=f"logits {lt} probs {qt}")


def test_empty_batch():
    case = linear_case(1, 3, 100, seed=1, dtype="f32")
    got = run_linear(case.logits[:0], case.draft_probs[:0], case.draft_tokens[:0], 1.0, 0)
    assert got["tokens"].shape == (0, 4)


def test_out_of_range_tokens_and_minus_inf():
    case = linear_case(16, 4, 512, seed=5, dtype="f32", noise_sigma=1.0)
    case.draft_tokens[:, 1] = torch.tensor([-1, 512, 10**6, -(10**6)] * 4, dtype=torch.int32)
    case.logits[:, :, 300:] = float("-inf")
    got, ref = _case_run(case, seed=3, what="invalid tokens and -inf logits")
    assert np.all(got["accept_len"] <= 1)
    assert np.all(got["tokens"][got["tokens"] >= 0] < 512)
    emitted = got["tokens"][np.arange(16), got["accept_len"]]
    assert np.all(emitted < 300)


def test_identical_draft_accepts_everything():
    case = linear_case(64, 6, 2000, seed=8, dtype="f32")
    L = to_numpy_f64(case.logits)
    z = L[:, :6] - L[:, :6].max(axis=-1, keepdims=True)
    p = np.exp(z) / np.exp(z).sum(axis=-1, keepdims=True)
    case.draft_probs = torch.from_numpy(p).to(torch.float32)
    got, ref = _case_run(case, seed=7, what="q = p")
    ok = ~ref["near_tie"]
    assert np.all(got["accept_len"][ok] == 6)


def test_disjoint_supports_emit_one():
    V, k = 64, 5
    p = np.zeros((k + 1, V))
    p[:, :32] = 1 / 32
    q = np.zeros((k, V))
    q[:, 32:] = 1 / 32
    case = fixed_pq_case(p, q, 500, seed=2, dtype="bf16")
    got, _ = _case_run(case, seed=8, what="disjoint supports")
    assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] < 32)


@pytest.mark.parametrize("lt,qt,V", [("bf16", "bf16", 70000),   # draft rows read in 16-byte vectors
                                     ("bf16", "bf16", 70001),   # element-wise
                                     ("f32", "bf16", 70000)])   # 8-byte bf16 chunks (LM-head path)
def test_residual_tiles_helped_by_later_rows(lt, qt, V):
    # Position 0 always rejects (disjoint supports): its residual is p_0 itself, over rows
    # walked in tiles (960 rows keep the batch off the split kernel).  The later rows of
    # each sequence stand down and sum some of those tiles for it.
    import speculative_sampling_verify_03_amd as sv
    k, B = 5, 160
    rng = np.random.default_rng(5)
    p = np.zeros((k + 1, V))
    p[:, : V // 2] = rng.uniform(0.5, 1.5, size=(k + 1, V // 2))
    p /= p.sum(axis=1, keepdims=True)
    q = np.zeros((k, V))
    q[:, V // 2:] = rng.uniform(0.5, 1.5, size=(k, V - V // 2))
    q /= q.sum(axis=1, keepdims=True)
    case = fixed_pq_case(p, q, B, seed=6, dtype=lt)
    case.draft_probs = case.draft_probs.to(torch.bfloat16 if qt == "bf16" else torch.float32)
    what = f"helped residual {lt}/{qt} V={V}"
    announce(what)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, B, k, V)
    for rep in range(2):  # the second call finds the help words cleared by the first
        got = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 9, rep, ws=ws)
        assert status_word(ws) == 0, f"{what}: a wait between workgroups ran out"
        assert sections_clear(ws, sv.SV_KIND_LINEAR, k, V)
        ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 9, rep)
        check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=V, what=f"{what} call {rep}")
        assert np.all(got["accept_len"] == 0) and np.all(got["tokens"][:, 0] < V // 2)


def test_deterministic_and_workspace_reuse():
    import speculative_sampling_verify_03_amd as sv
    case = linear_case(64, 5, 32000, seed=21, dtype="bf16", noise_sigma=0.7)
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, 64, 5, 32000)
    a = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 3, 0, ws=ws)
    b = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 3, 0, ws=ws)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    assert int(ws[:64 * 4].view(torch.int32).abs().sum()) == 0  # tickets back to zero
    c = run_linear(case.logits[:10], case.draft_probs[:10], case.draft_tokens[:10], 1.0, 3, 0, ws=ws)
    assert np.array_equal(c["tokens"], a["tokens"][:10])


@pytest.mark.parametrize("what", ["single-tile", "multi-tile", "every row rejects"])
def test_workspace_returns_to_zero(what):
    # Row kernel: rejected rows post their position to a per-sequence word before drawing,
    # and the finishing workgroup clears it after every row's ticket: the whole workspace
    # must be zero after a call, so that the next call starts clean (and so must its
    # results).  The single- and multi-tile cases here take the split kernel, whose tagged
    # words stay in the workspace's prefix; everything after it must be zero either way.
    import speculative_sampling_verify_03_amd as sv
    if what == "single-tile":
        case = linear_case(64, 5, 32000, seed=31, dtype="bf16", noise_sigma=1.5)
    elif what == "multi-tile":
        case = linear_case(24, 4, 70001, seed=32, dtype="bf16", noise_sigma=1.5)
    else:
        V, k = 64, 5
        p = np.zeros((k + 1, V))
        p[:, :32] = 1 / 32
        q = np.zeros((k, V))
        q[:, 32:] = 1 / 32
        case = fixed_pq_case(p, q, 300, seed=3, dtype="bf16")
    announce(f"workspace clean-up: {what} B={case.B} k={case.k} V={case.V}")
    ws = sv.new_workspace(sv.SV_KIND_LINEAR, case.B, case.k, case.V)
    ref = oracle_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 9, 0)
    for rep in range(2):
        got = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 9, 0, ws=ws)
        assert status_word(ws) == 0, f"call {rep}: a wait between workgroups ran out"
        assert sections_clear(ws, sv.SV_KIND_LINEAR, case.k, case.V), f"call {rep}: workspace not cleared"
        check_linear(got, ref, case.logits.dtype, X=case.draft_tokens.numpy(), V=case.V,
                     what=f"{what} call {rep}")
    assert (ref["accept_len"] < case.k).sum() > 0  # the case has rejections


def test_chisquare_gpu_output_law():
    """1e6 sequences, V = 8: tokens emitted at each reached position follow p_j."""
    rng = np.random.default_rng(31)
    V, k = 8, 2
    p = rng.dirichlet(np.ones(V), size=k + 1)
    q = rng.dirichlet(np.ones(V), size=k)
    B = 1_000_000
    case = fixed_pq_case(p, q, B, seed=31, dtype="f32")
    announce("chi-square: B=1e6 V=8 k=2")
    got = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 77, 0)
    # the kernel's own target law is softmax of the float32 logits; compare against p
    for j in range(k + 1):
        reached = got["accept_len"] >= j
        counts = np.bincount(got["tokens"][reached, j], minlength=V)
        pv = stats.chisquare(counts, p[j] * reached.sum()).pvalue
        announce(f"position {j}: reached {reached.sum()}, chi-square p-value {pv:.3g}")
        assert pv > 1e-3


@pytest.mark.parametrize("alpha", [0.3, 0.75, 0.9])
def test_closed_form_on_gpu(alpha):
    V, k = 8, 4
    q = np.array([0.25, 0.25, 0.25, 0.25, 0, 0, 0, 0])
    p = alpha * q
    p[7] += 1 - alpha
    B = 400_000
    case = fixed_pq_case(np.tile(p, (k + 1, 1)), np.tile(q, (k, 1)), B, seed=int(alpha * 10), dtype="f32")
    got = run_linear(case.logits, case.draft_probs, case.draft_tokens, 1.0, 5, 0)
    emitted = got["accept_len"] + 1.0
    expect = (1 - alpha ** (k + 1)) / (1 - alpha)
    se = emitted.std() / np.sqrt(B)
    announce(f"alpha={alpha}: mean emitted {emitted.mean():.5f} vs closed form {expect:.5f} (se {se:.2g})")
    assert abs(emitted.mean() - expect) < 4 * se
