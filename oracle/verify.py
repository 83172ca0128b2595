"""Verification / speculative-sampling step, written out plainly in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Inputs are numpy arrays holding
the exact values the device sees (float32 or bfloat16 widened to float64); every
intermediate is float64.  One sequence at a time, one position at a time.

What the pages fix, and the readings taken where they are silent:

* The target model gives, at every position of the drafted sequence, the probability
  distribution of the next token (*Sonar*, section "Speculative decoding").  Reading:
  p_j = softmax(l_j / T), temperature T > 0 applied to the target logits only.
* Acceptance (*Explained*, section "Draft and verification loop"): a draft token is
  kept outright when the target is at least as confident in it as the draft was,
  otherwise it is kept with a probability that falls as the gap grows, and on
  rejection a corrected token is drawn from an adjusted distribution; the result has
  the target's distribution exactly.  Reading: keep x with probability min(1, p(x)/q(x)),
  evaluated as ``u_acc * q(x) < p(x)`` (strict, no division; q(x) = 0 accepts iff
  p(x) > 0); the adjusted distribution is the normalised residual max(0, p - q).
* The sampler fixes the longest acceptable prefix (*Sonar*, section "Speculative
  decoding", acceptance stage), and the target's logits at the mismatch or at the end of
  the draft give one more token for free (same section, target-generation stage;
  *Explained*, section "Best and worst case": up to k+1 tokens per pass, exactly one in
  the worst case).  Reading: n = first rejected position (k if none); emit the n
  accepted drafts, then a residual draw at row n if n < k or a draw from p_k if n = k.
* Draws: ``oracle.philox.uniforms(seed, seq=b, pos=j, offset)``.  Inverse-CDF sampling
  over ascending token ids: the smallest i with C_i > u * S, C the running sum of the
  weights and S their total.
* Residual mass S = 0 can only come from rounding (p <= q everywhere forces p = q, and
  then nothing is rejected in exact arithmetic).  Reading: fall back to p_n.
* Greedy variant: target argmax (first index of the maximum of the raw logits) must
  equal the draft token; the bonus/correction token is the target argmax at row n.
* Static tree (*Sonar*, section "EAGLE": a static tree of draft tokens is explored and
  the longest acceptable sequence wins, plus one target token).  Reading: node c with
  parent u is tested against rows u of the target and draft distributions with the
  draw at pos = c; a node is alive when it and all its ancestors pass; the chosen node
  is the deepest alive node, lowest BFS index on ties (leftmost path); the extra token
  is drawn from p at the chosen node (no residual -- this variant does not keep the
  exact target law; *Explained*, section "Variants without a separate draft model",
  notes such trade-offs).
* Draft tokens outside [0, V) are rejected with p(x) = 0 and q(x) never read.
"""
from __future__ import annotations

import numpy as np

from .philox import uniforms

NEAR_TIE = 1e-6


def _draws(seed: int, seq: int, pos: int, offset: int, u_shift=(0.0, 0.0)):
    """(u_acc, u_smp) of one position, each moved by u_shift and kept inside [0, 1).

    u_shift is a test hook (default: no shift): moving every draw of a sequence by about
    the near-tie width shows which outcomes a near-tie decision can take.
    """
    u_acc, u_smp = uniforms(seed, seq, pos, offset)
    top = 1.0 - 2.0 ** -53
    return (min(max(u_acc + u_shift[0], 0.0), top), min(max(u_smp + u_shift[1], 0.0), top))


def target_distribution(logit_row, temperature: float) -> np.ndarray:
    """p = softmax(l / T) over one vocabulary row, float64."""
    z = np.asarray(logit_row, dtype=np.float64) / float(temperature)
    m = np.max(z)
    e = np.exp(z - m)
    return e / np.sum(e)


def inverse_cdf_sample(w: np.ndarray, u: float):
    """Draw from the (unnormalised, non-negative) weights w with the uniform u.

    Returns (y, margin): y is the smallest index i with C_i > u * S where C is the
    ascending running sum of w and S = C[-1]; margin is the distance of u from the two
    normalised CDF values bracketing y, min(|u - C_{y-1}/S|, |u - C_y/S|).
    Requires S > 0.
    """
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    S = C[-1]
    assert S > 0.0
    t = u * S
    y = int(np.searchsorted(C, t, side="right"))
    if y >= C.shape[0]:
        y = int(np.nonzero(w > 0)[0][-1])
    lo = C[y - 1] / S if y > 0 else 0.0
    hi = C[y] / S
    return y, min(abs(u - lo), abs(u - hi))


def acceptance_overlap(p: np.ndarray, q: np.ndarray) -> float:
    """Probability that a draft token x ~ q passes the test against p: sum_v min(p, q)."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def _accept(u_acc: float, px: float, qx: float):
    """The acceptance comparison and its distance from the threshold u = p/q."""
    acc = u_acc * qx < px
    margin = abs(u_acc - px / qx) if qx > 0.0 else np.inf
    if qx > 0.0:
        aprob = min(1.0, px / qx)
    else:
        aprob = 1.0 if px > 0.0 else 0.0
    return acc, margin, aprob


def verify_linear(logits, draft_probs, draft_tokens, temperature: float, seed: int,
                  offset: int = 0, seq_base: int = 0, u_shift=(0.0, 0.0)):
    """Linear speculative sampling.

    logits [B, k+1, V], draft_probs [B, k, V], draft_tokens [B, k] int.  Sequence b
    draws with sequence id seq_base + b (seq_base lets a caller verify one sequence of a
    batch on its own); u_shift is the test hook of _draws.
    Returns a dict of numpy arrays:
      tokens [B, k+1] (emitted tokens, -1 padded), accept_len [B] (= n, drafts kept;
      emitted = n + 1), target_prob [B, k] (p_j(x_j)), accept_prob [B, k]
      (min(1, p/q)), accepted [B, k] (every position's test), fallback [B] (S = 0 path),
      residual_mass [B] (S of the final draw's weights: the residual mass, or 1 for a
      draw from p), acc_margin / smp_margin [B] (distance of the deciding draws from
      their thresholds) and near_tie [B] (either margin below 1e-6).
    """
    L = np.asarray(logits, dtype=np.float64)
    Q = np.asarray(draft_probs, dtype=np.float64)
    X = np.asarray(draft_tokens, dtype=np.int64)
    B, R, V = L.shape
    k = R - 1
    out = dict(
        tokens=np.full((B, R), -1, dtype=np.int32),
        accept_len=np.zeros(B, dtype=np.int32),
        target_prob=np.zeros((B, k), dtype=np.float64),
        accept_prob=np.zeros((B, k), dtype=np.float64),
        accepted=np.zeros((B, k), dtype=bool),
        fallback=np.zeros(B, dtype=bool),
        residual_mass=np.ones(B, dtype=np.float64),
        acc_margin=np.full(B, np.inf),
        smp_margin=np.full(B, np.inf),
    )
    for b in range(B):
        p = [target_distribution(L[b, j], temperature) for j in range(R)]
        n = k
        for j in range(k):
            u_acc, _ = _draws(seed, seq_base + b, j, offset, u_shift)
            x = int(X[b, j])
            if 0 <= x < V:
                acc, margin, aprob = _accept(u_acc, p[j][x], Q[b, j, x])
                out["target_prob"][b, j] = p[j][x]
                out["accept_prob"][b, j] = aprob
            else:
                acc, margin = False, np.inf
            out["accepted"][b, j] = acc
            if n == k:  # decisions up to and including the first rejection decide n
                out["acc_margin"][b] = min(out["acc_margin"][b], margin)
                if not acc:
                    n = j
        _, u_smp = _draws(seed, seq_base + b, n, offset, u_shift)
        if n < k:
            w = np.maximum(0.0, p[n] - Q[b, n])
            if np.sum(w) == 0.0:
                w = p[n]
                out["fallback"][b] = True
            else:
                out["residual_mass"][b] = np.sum(w)
        else:
            w = p[k]
        y, smargin = inverse_cdf_sample(w, u_smp)
        out["smp_margin"][b] = smargin
        out["accept_len"][b] = n
        out["tokens"][b, :n] = X[b, :n]
        out["tokens"][b, n] = y
    out["near_tie"] = (out["acc_margin"] < NEAR_TIE) | (out["smp_margin"] < NEAR_TIE)
    return out


def verify_greedy(logits, draft_tokens):
    """Greedy verification: accept while the target argmax equals the draft token.

    Returns tokens [B, k+1] (-1 padded), accept_len [B] and argmax [B, k+1] (first index
    of the maximum raw logit of every row).
    """
    L = np.asarray(logits, dtype=np.float64)
    X = np.asarray(draft_tokens, dtype=np.int64)
    B, R, _ = L.shape
    k = R - 1
    g = np.argmax(L, axis=-1).astype(np.int32)  # numpy returns the first maximum
    tokens = np.full((B, R), -1, dtype=np.int32)
    acc_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = k
        for j in range(k):
            if g[b, j] != X[b, j]:
                n = j
                break
        acc_len[b] = n
        tokens[b, :n] = X[b, :n]
        tokens[b, n] = g[b, n]
    return dict(tokens=tokens, accept_len=acc_len, argmax=g)


def tree_depths(parents) -> np.ndarray:
    par = np.asarray(parents, dtype=np.int64)
    d = np.zeros(par.shape[0], dtype=np.int32)
    for c in range(1, par.shape[0]):
        d[c] = d[par[c]] + 1
    return d


def verify_tree(logits, draft_probs, node_tokens, parents, temperature: float, seed: int,
                offset: int = 0, seq_base: int = 0, u_shift=(0.0, 0.0)):
    """Static-tree verification.

    logits [B, N, V] (row u: target distribution after the path to node u),
    draft_probs [B, N, V] (row u: draft distribution from which u's children came),
    node_tokens [B, N] (entry 0, the root, unused), parents [N] (BFS order, parents[0]
    = -1, 0 <= parents[c] < c).
    Returns tokens [B, D+1] and path [B, D+1] (node ids root..chosen, -1 padded) with D
    the tree depth, accept_len [B] (depth of the chosen node), chosen [B], accepted and
    alive [B, N], acc_margin / smp_margin / near_tie [B].  seq_base and u_shift: as for
    verify_linear.
    """
    L = np.asarray(logits, dtype=np.float64)
    Q = np.asarray(draft_probs, dtype=np.float64)
    T_ = np.asarray(node_tokens, dtype=np.int64)
    par = np.asarray(parents, dtype=np.int64)
    B, N, V = L.shape
    depth = tree_depths(par)
    D = int(depth.max())
    out = dict(
        tokens=np.full((B, D + 1), -1, dtype=np.int32),
        path=np.full((B, D + 1), -1, dtype=np.int32),
        accept_len=np.zeros(B, dtype=np.int32),
        chosen=np.zeros(B, dtype=np.int32),
        accepted=np.zeros((B, N), dtype=bool),
        alive=np.zeros((B, N), dtype=bool),
        acc_margin=np.full(B, np.inf),
        smp_margin=np.full(B, np.inf),
    )
    for b in range(B):
        p = {}

        def prow(u):
            if u not in p:
                p[u] = target_distribution(L[b, u], temperature)
            return p[u]

        alive = np.zeros(N, dtype=bool)
        alive[0] = True
        out["accepted"][b, 0] = True
        for c in range(1, N):
            u = int(par[c])
            x = int(T_[b, c])
            u_acc, _ = _draws(seed, seq_base + b, c, offset, u_shift)
            if 0 <= x < V:
                acc, margin, _ = _accept(u_acc, prow(u)[x], Q[b, u, x])
            else:
                acc, margin = False, np.inf
            out["accepted"][b, c] = acc
            alive[c] = alive[u] and acc
            if alive[u]:  # only tests under a live parent can change the outcome
                out["acc_margin"][b] = min(out["acc_margin"][b], margin)
        out["alive"][b] = alive
        best = 0
        for c in range(1, N):
            if alive[c] and depth[c] > depth[best]:
                best = c
        chain = [best]
        while chain[-1] != 0:
            chain.append(int(par[chain[-1]]))
        chain.reverse()
        _, u_smp = _draws(seed, seq_base + b, best, offset, u_shift)
        y, smargin = inverse_cdf_sample(prow(best), u_smp)
        d = int(depth[best])
        out["chosen"][b] = best
        out["accept_len"][b] = d
        out["path"][b, :d + 1] = chain
        out["tokens"][b, :d] = [T_[b, c] for c in chain[1:]]
        out["tokens"][b, d] = y
        out["smp_margin"][b] = smargin
    out["near_tie"] = (out["acc_margin"] < NEAR_TIE) | (out["smp_margin"] < NEAR_TIE)
    return out


def lmhead_logits(hidden, weight) -> np.ndarray:
    """Target logits from final hidden states and the LM-head weight [H, V], float64.

    *Sonar*, sections "EAGLE" and "Training MTP heads": the heads reuse the target's
    LM head (about 2 GB in bf16 for a 70B model), so the logits that verification
    consumes are hidden @ W.
    """
    h = np.asarray(hidden, dtype=np.float64)
    return h @ np.asarray(weight, dtype=np.float64)


def lmhead_gemm_error_bound(hidden, weight) -> np.ndarray:
    """Entrywise bound on |fp32-accumulated hidden @ W - exact| for bf16 inputs.

    Products of two bf16 values are exact in float32, so only the K additions round:
    |error| <= gamma_K * sum_h |a_h w_hv| with gamma_K = K u / (1 - K u), u = 2^-24
    (Higham, Accuracy and Stability of Numerical Algorithms, section 3.1).  Twice that,
    to cover any summation order and the final conversion.
    """
    h = np.abs(np.asarray(hidden, dtype=np.float64))
    w = np.abs(np.asarray(weight, dtype=np.float64))
    K = h.shape[-1]
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    return 2.0 * gamma * (h @ w)


def lmhead_gemm_error_bound_probabilistic(hidden, weight, lam: float = 10.0) -> np.ndarray:
    """Entrywise probabilistic bound on |fp32-accumulated hidden @ W - exact|.

    Higham and Mary, "A new approach to probabilistic rounding error analysis" (SIAM J.
    Sci. Comput. 41(5), 2019): if the rounding errors of the K additions are independent,
    mean-zero and at most u in size, the computed inner product is within
    gamma(lam) * sum_h |a_h w_hv| of the exact one, gamma(lam) = exp(lam sqrt(K) u +
    K u^2 / (1 - u)) - 1, except with probability at most 2 K exp(-lam^2 (1 - u)^2 / 2).
    lam = 10 at K = 8192: at most 3.1e-18 per entry; the bound is about 1/18 of the
    worst-case one (lmhead_gemm_error_bound) there, tight enough that leaving out one
    product a_h * w_hv of typical size exceeds it.  Products of bf16 values are exact in
    float32, so only the additions round.
    """
    h = np.abs(np.asarray(hidden, dtype=np.float64))
    w = np.abs(np.asarray(weight, dtype=np.float64))
    K = h.shape[-1]
    u = 2.0 ** -24
    gamma = np.expm1(lam * np.sqrt(K) * u + K * u * u / (1.0 - u))
    return gamma * (h @ w)


def verify_lmhead(hidden, weight, draft_probs, draft_tokens, temperature: float,
                  seed: int, offset: int = 0):
    """LM-head projection followed by linear verification.

    hidden [B, k+1, H], weight [H, V]."""
    return verify_linear(lmhead_logits(hidden, weight), draft_probs, draft_tokens,
                         temperature, seed, offset)
