"""Seeded generators for the verification workloads.

Every generator draws from ``numpy.random.default_rng(seed)`` in a fixed order, so a
(seed, shape) pair always yields the same tensors.  Tensors come back on the CPU as
torch tensors in the dtype the verification step consumes (float32 or bfloat16 via
torch's round-to-nearest-even cast) plus int32 token ids.

The workloads follow the shapes the source pages talk about: Llama-class vocabularies
(32000, 128256), hidden size 8192 with a ~2 GB bf16 LM head ("Accelerating Sonar
through speculation", section "Training MTP heads"), 4-8 draft tokens per step
("Speculative decoding explained", section "Draft and verification loop"), and an
EAGLE-style static tree (Sonar post, section "EAGLE").

What is generated here is the *draft side* of speculative decoding (draft logits,
the draft's own softmax, draft tokens drawn from it) and the target's raw logits.  The
target-side arithmetic of the verification step lives elsewhere.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# Noise scale between draft and target logits for the B=64, k=5, V=32000 workload.
# Chosen so that the mean per-position acceptance probability sum_v min(p, q) over the
# seed-2 batch is 0.75 (the middle of the 70-80% range quoted in "Speculative decoding
# explained", section "Best and worst case"): a bisection over sigma of that mean,
# twelve halvings of [0.3, 1.2].  A CPU test holds the mean at 0.75 +- 0.005.
CFG2_NOISE_SIGMA = 0.6483764648

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Case:
    """Inputs of one linear (or greedy) verification call."""
    logits: torch.Tensor         # [B, k+1, V] target logits (f32 or bf16)
    draft_probs: torch.Tensor    # [B, k, V] draft probabilities (f32 or bf16)
    draft_tokens: torch.Tensor   # int32 [B, k], sampled from draft_probs
    greedy_tokens: torch.Tensor  # int32 [B, k], argmax of the draft logits
    temperature: float
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.logits.shape[0]

    @property
    def k(self):
        return self.logits.shape[1] - 1

    @property
    def V(self):
        return self.logits.shape[2]


@dataclass
class TreeCase:
    logits: torch.Tensor        # [B, N, V]; row u = target logits after the path to node u
    draft_probs: torch.Tensor   # [B, N, V]; row u = draft distribution of u's children
    node_tokens: torch.Tensor   # int32 [B, N]; entry 0 (root) unused (set to 0)
    parents: np.ndarray         # int32 [N]; parents[0] = -1, BFS order
    temperature: float
    meta: dict = field(default_factory=dict)


@dataclass
class LMHeadCase:
    hidden: torch.Tensor        # bf16 [B, k+1, H]
    weight: torch.Tensor        # bf16 [H, V], row-major
    draft_probs: torch.Tensor   # [B, k, V]
    draft_tokens: torch.Tensor  # int32 [B, k]
    temperature: float
    meta: dict = field(default_factory=dict)


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a float32 / bfloat16 tensor (both widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.array(a, dtype=np.float64, order="C")).to(_TORCH_DTYPES[dtype])


def _draft_softmax(d: np.ndarray, temp: float = 1.0) -> np.ndarray:
    """The draft model's own output distribution over the last axis (float64)."""
    s = d.astype(np.float64) / temp
    s = s - s.max(axis=-1, keepdims=True)
    np.exp(s, out=s)
    s /= s.sum(axis=-1, keepdims=True)
    return s


def _draw_tokens(rng: np.random.Generator, q_cast: torch.Tensor) -> np.ndarray:
    """Draft tokens drawn from the probabilities as the verifier will see them.

    Each row of the cast draft probabilities is renormalised in float64 and passed to
    ``Generator.choice``; rows are visited in C order.
    """
    q = to_numpy_f64(q_cast)
    flat = q.reshape(-1, q.shape[-1])
    out = np.empty(flat.shape[0], dtype=np.int32)
    V = flat.shape[1]
    for r in range(flat.shape[0]):
        row = flat[r] / flat[r].sum()
        out[r] = rng.choice(V, p=row)
    return out.reshape(q.shape[:-1])


def linear_case(B: int, k: int, V: int, *, seed: int, dtype: str = "bf16",
                draft_sigma: float = 2.0, noise_sigma: float = 0.5,
                temperature: float = 1.0, boost_frac: float = 0.0,
                boost: float = 8.0) -> Case:
    """Draft logits D ~ N(0, draft_sigma^2) of shape [B, k+1, V]; with probability
    ``boost_frac`` a (b, j) row gets ``boost`` added at one uniform token; target logits
    are D + N(0, noise_sigma^2); draft probabilities are softmax(D / temperature) on the
    first k rows; draft tokens are drawn from them.  Generated one sequence at a time.
    """
    R = k + 1
    rng = np.random.default_rng(seed)
    tdt = _TORCH_DTYPES[dtype]
    logits = torch.empty((B, R, V), dtype=tdt)
    probs = torch.empty((B, k, V), dtype=tdt)
    greedy = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        d = rng.standard_normal((R, V), dtype=np.float32).astype(np.float64) * draft_sigma
        if boost_frac > 0.0:
            hit = rng.random(R) < boost_frac
            tok = rng.integers(0, V, size=R)
            d[hit, tok[hit]] += boost
        noise = rng.standard_normal((R, V), dtype=np.float32).astype(np.float64) * noise_sigma
        logits[b] = _cast(d + noise, dtype)
        if k > 0:
            probs[b] = _cast(_draft_softmax(d[:k], temperature), dtype)
            greedy[b] = np.argmax(d[:k], axis=-1)
    tokens = _draw_tokens(rng, probs) if k > 0 else np.zeros((B, 0), np.int32)
    return Case(logits=logits, draft_probs=probs,
                draft_tokens=torch.from_numpy(tokens.astype(np.int32)),
                greedy_tokens=torch.from_numpy(greedy), temperature=temperature,
                meta=dict(seed=seed, dtype=dtype, draft_sigma=draft_sigma,
                          noise_sigma=noise_sigma, boost_frac=boost_frac))


def cfg1_case(B: int = 1, seed: int = 1) -> Case:
    """B=1 (or batched), k=4, V=1024, float32, T=1: D ~ N(0, 2^2), target = D + N(0, 0.5^2)."""
    return linear_case(B, 4, 1024, seed=seed, dtype="f32", draft_sigma=2.0, noise_sigma=0.5)


def cfg2_case(seed: int = 2, B: int = 64) -> Case:
    """B=64, k=5, V=32000, bf16: D ~ N(0, 3^2) with 5% of rows boosted by +8 at one
    token, target = D + N(0, sigma^2) with sigma tuned for ~75% acceptance."""
    return linear_case(B, 5, 32000, seed=seed, dtype="bf16", draft_sigma=3.0,
                       noise_sigma=CFG2_NOISE_SIGMA, boost_frac=0.05, boost=8.0)


def cfg3_case(seed: int = 3, B: int = 256) -> Case:
    """B=256, k=8, V=128256, bf16, T=0.7 with the cfg1 generator (draft probs at T=0.7)."""
    return linear_case(B, 8, 128256, seed=seed, dtype="bf16", draft_sigma=2.0,
                       noise_sigma=0.5, temperature=0.7)


def mtp_case(seed: int = 6, B: int = 256) -> Case:
    """Single-token MTP regime of "Accelerating Sonar through speculation" (section "MTP
    schedule for one token": one drafted token per sequence, the target checks 2 tokens per
    sequence): B=256, k=1, V=128256, bf16, T=1, cfg1-style logits."""
    return linear_case(B, 1, 128256, seed=seed, dtype="bf16", draft_sigma=2.0, noise_sigma=0.5,
                       temperature=1.0)


def eagle_tree_parents(branching=(4, 2, 2, 2), max_nodes: int = 61) -> np.ndarray:
    """Parent array of a static tree in BFS order: the root has branching[0] children,
    every node of level d has branching[d] children, truncated to ``max_nodes`` slots
    (root included).  (4, 2, 2, 2) gives 1 + 4 + 8 + 16 + 32 = 61 nodes."""
    parents = [-1]
    level = [0]
    for br in branching:
        nxt = []
        for u in level:
            for _ in range(br):
                if len(parents) >= max_nodes:
                    break
                parents.append(u)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.asarray(parents[:max_nodes], dtype=np.int32)


def chain_tree_parents(n: int) -> np.ndarray:
    """A chain: node i's parent is i-1 (a linear draft written as a tree)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_case(B: int, parents: np.ndarray, V: int, *, seed: int, dtype: str = "bf16",
              draft_sigma: float = 2.0, noise_sigma: float = 0.5,
              temperature: float = 1.0, sample_children: bool = False) -> TreeCase:
    """Per node u: D_u ~ N(0, draft_sigma^2), target row = D_u + N(0, noise_sigma^2),
    draft row = softmax(D_u).  The children of u take the top tokens of u's draft row in
    descending order (lowest id on ties), or, with ``sample_children``, tokens drawn
    from it."""
    parents = np.asarray(parents, dtype=np.int32)
    N = parents.shape[0]
    rng = np.random.default_rng(seed)
    tdt = _TORCH_DTYPES[dtype]
    logits = torch.empty((B, N, V), dtype=tdt)
    probs = torch.empty((B, N, V), dtype=tdt)
    toks = np.zeros((B, N), dtype=np.int32)
    children = [[] for _ in range(N)]
    for c in range(1, N):
        children[parents[c]].append(c)
    for b in range(B):
        d = rng.standard_normal((N, V), dtype=np.float32).astype(np.float64) * draft_sigma
        noise = rng.standard_normal((N, V), dtype=np.float32).astype(np.float64) * noise_sigma
        logits[b] = _cast(d + noise, dtype)
        qc = _cast(_draft_softmax(d, temperature), dtype)
        probs[b] = qc
        q64 = to_numpy_f64(qc)
        for u in range(N):
            ch = children[u]
            if not ch:
                continue
            if sample_children:
                row = q64[u] / q64[u].sum()
                picks = rng.choice(V, size=len(ch), p=row)
            else:
                order = np.argsort(-q64[u], kind="stable")
                picks = order[:len(ch)]
            for c, t in zip(ch, picks):
                toks[b, c] = t
    return TreeCase(logits=logits, draft_probs=probs, node_tokens=torch.from_numpy(toks),
                    parents=parents, temperature=temperature,
                    meta=dict(seed=seed, dtype=dtype))


def cfg5_case(seed: int = 5, B: int = 16) -> TreeCase:
    """B=16, 61-node static tree (top-4 then top-2), V=128256, bf16, T=1."""
    return tree_case(B, eagle_tree_parents(), 128256, seed=seed, dtype="bf16")


def lmhead_case(B: int, k: int, H: int, V: int, *, seed: int, dtype: str = "bf16",
                w_sigma: float = 0.02, draft_noise: float = 1.0,
                temperature: float = 1.0) -> LMHeadCase:
    """hidden ~ N(0, 1) bf16 [B, k+1, H]; W ~ N(0, w_sigma^2) bf16 [H, V].  The draft
    logits are the first k rows' hidden @ W (float32 matmul of the bf16 values, a
    stand-in for a draft head that tracks the target) plus N(0, draft_noise^2); draft
    probabilities are their softmax; draft tokens are drawn from them."""
    rng = np.random.default_rng(seed)
    R = k + 1
    hidden = torch.from_numpy(rng.standard_normal((B, R, H), dtype=np.float32)).to(torch.bfloat16)
    w = torch.empty((H, V), dtype=torch.bfloat16)
    step = 1024
    for h0 in range(0, H, step):
        h1 = min(H, h0 + step)
        blk = rng.standard_normal((h1 - h0, V), dtype=np.float32)
        blk *= np.float32(w_sigma)
        w[h0:h1] = torch.from_numpy(blk).to(torch.bfloat16)
    probs = torch.empty((B, k, V), dtype=_TORCH_DTYPES[dtype])
    if k > 0:
        hd = hidden[:, :k, :].reshape(B * k, H).to(torch.float32)
        dl = (hd @ w.to(torch.float32)).to(torch.float64).numpy().reshape(B, k, V)
        dl += rng.standard_normal((B, k, V), dtype=np.float32).astype(np.float64) * draft_noise
        probs[:] = _cast(_draft_softmax(dl, temperature), dtype)
    tokens = _draw_tokens(rng, probs) if k > 0 else np.zeros((B, 0), np.int32)
    return LMHeadCase(hidden=hidden, weight=w, draft_probs=probs,
                      draft_tokens=torch.from_numpy(tokens.astype(np.int32)),
                      temperature=temperature, meta=dict(seed=seed))


def cfg4_case(seed: int = 4, B: int = 32) -> LMHeadCase:
    """B=32, k=5, H=8192, V=128256: the Llama-70B-shaped LM head feeding verification."""
    return lmhead_case(B, 5, 8192, 128256, seed=seed)


def fixed_pq_case(p: np.ndarray, q: np.ndarray, B: int, *, seed: int,
                  dtype: str = "f32") -> Case:
    """B independent sequences sharing fixed target distributions p [k+1, V] and draft
    distributions q [k, V].  Target logits are log p (T = 1); draft tokens are drawn
    from q for every sequence independently."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    R, V = p.shape
    k = R - 1
    rng = np.random.default_rng(seed)
    with np.errstate(divide="ignore"):
        lp = np.log(p)
    logits = _cast(np.broadcast_to(lp, (B, R, V)), dtype)
    probs = _cast(np.broadcast_to(q, (B, k, V)), dtype)
    qv = to_numpy_f64(probs[0]) if k > 0 else np.zeros((0, V))
    toks = np.zeros((B, k), dtype=np.int32)
    for j in range(k):
        row = qv[j] / qv[j].sum()
        toks[:, j] = rng.choice(V, size=B, p=row)
    greedy = np.tile(np.argmax(q, axis=-1).astype(np.int32), (B, 1)) if k > 0 else toks
    return Case(logits=logits, draft_probs=probs, draft_tokens=torch.from_numpy(toks),
                greedy_tokens=torch.from_numpy(greedy), temperature=1.0,
                meta=dict(seed=seed, dtype=dtype))


def lookup_histories(B: int, cap: int, vocab: int = 32000, seed: int = 0, doc_frac: float = 0.7):
    """Token histories for prompt lookup, standing in for the page's code-editing and
    summarisation prompts: a random "document" of about doc_frac * cap tokens, then a
    "response" that copies spans of 4-32 tokens from it with one token in ten replaced at
    random.  Lengths vary between cap/2 and cap.  Returns (history int64 [B, cap] with -1
    past each length, lengths int64 [B])."""
    rng = np.random.default_rng(seed)
    hist = np.full((B, cap), -1, dtype=np.int64)
    lens = rng.integers(max(1, cap // 2), cap + 1, size=B)
    for b in range(B):
        L = int(lens[b])
        nd = max(1, int(L * doc_frac))
        doc = rng.integers(0, vocab, size=nd)
        out = list(doc)
        while len(out) < L:
            s = int(rng.integers(0, nd))
            span = list(doc[s:s + int(rng.integers(4, 33))])
            for i in range(len(span)):
                if rng.random() < 0.1:
                    span[i] = int(rng.integers(0, vocab))
            out += span
        hist[b, :L] = np.array(out[:L], dtype=np.int64)
    return hist, lens
