"""Lossless static-tree verification: the siblings of a node are tried in order against
the target distribution left after the earlier siblings' rejections.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's CPU
baseline, never by the product path.

What the pages fix: the tree holds the top-K draft candidates at every node and the
longest acceptable sequence wins, plus one target token (*Sonar*, section "EAGLE"); some
tree and draft variants give up the exact target law (*Explained*, section "Variants
without a separate draft model"), while the basic test keeps it (*Explained*, section
"Draft and verification loop").  The pages give no procedure for keeping the law with
several candidates per node.

Reading (the plainest rule that keeps the target law with fixed candidates): the
candidates at a node are deterministic (the top-K of the draft), so each is a draft
distribution concentrated on one token.  Walking from the root, at node u with children
c_1..c_m (BFS order = draft rank) and target p = p_u:
  * W_i = 1 - (sum of p over the distinct valid tokens of c_1..c_{i-1}), summed in
    sibling order: the mass left after removing the rejected siblings;
  * c_i is kept iff its token x is valid (0 <= x < V), not a repeat of an earlier
    sibling's token, and u_acc * W_i < p(x) (probability p(x) / W_i, the basic test with
    the one-token draft against the renormalised remainder), with
    u_acc = uniforms(seed, b, c_i, offset)[0];
  * the first kept child is the next node (its token is emitted); if none is kept, the
    extra token is drawn from p with the children's tokens removed (inverse CDF over
    ascending ids, u_smp = uniforms(seed, b, u, offset)[1]); a node without children
    draws from p itself.  A remainder of zero mass (only through rounding) draws from p.
So P(emit c_i) = W_i * p(c_i) / W_i = p(c_i), and a token outside the children has
probability W_{m+1} * p(x) / W_{m+1} = p(x): every emitted token follows the target.
"""
from __future__ import annotations

import numpy as np

from .verify import NEAR_TIE, _draws, inverse_cdf_sample, target_distribution, tree_depths


def verify_tree_lossless(logits, node_tokens, parents, temperature: float, seed: int, offset: int = 0,
                         seq_base: int = 0, u_shift=(0.0, 0.0)):
    """logits [B, N, V] (row u: target distribution after the path to node u), node_tokens
    [B, N] (entry 0 unused), parents [N] (BFS order, parents[0] = -1).  Sequence b draws
    with sequence id seq_base + b; u_shift moves every draw (a test hook, default none).
    Returns tokens [B, D+1], path [B, D+1] (node ids, -1 padded), accept_len [B],
    chosen [B], acc_margin / smp_margin / near_tie [B], fallback [B]."""
    L = np.asarray(logits, dtype=np.float64)
    X = np.asarray(node_tokens, dtype=np.int64)
    par = np.asarray(parents, dtype=np.int64)
    B, N, V = L.shape
    depth = tree_depths(par)
    D = int(depth.max())
    children = [[c for c in range(1, N) if par[c] == u] for u in range(N)]
    out = dict(
        tokens=np.full((B, D + 1), -1, dtype=np.int32),
        path=np.full((B, D + 1), -1, dtype=np.int32),
        accept_len=np.zeros(B, dtype=np.int32),
        chosen=np.zeros(B, dtype=np.int32),
        acc_margin=np.full(B, np.inf),
        smp_margin=np.full(B, np.inf),
        fallback=np.zeros(B, dtype=bool),
    )
    for b in range(B):
        u = 0
        path = [0]
        while True:
            p = target_distribution(L[b, u], temperature)
            removed = []          # distinct valid tokens of the rejected siblings, in order
            before = 0.0          # their mass, summed in sibling order
            nxt = -1
            for c in children[u]:
                x = int(X[b, c])
                u_acc, _ = _draws(seed, seq_base + b, c, offset, u_shift)
                if not (0 <= x < V) or x in removed:
                    continue      # rejected; removes nothing new
                W = 1.0 - before
                px = p[x]
                acc = W > 0.0 and u_acc * W < px
                if W > 0.0:
                    out["acc_margin"][b] = min(out["acc_margin"][b], abs(u_acc - px / W))
                if acc:
                    nxt = c
                    break
                removed.append(x)
                before += px
            if nxt < 0:
                break
            u = nxt
            path.append(u)
        p = target_distribution(L[b, u], temperature)
        w = p.copy()
        w[removed] = 0.0
        if np.sum(w) == 0.0:
            w = p
            out["fallback"][b] = True
        _, u_smp = _draws(seed, seq_base + b, u, offset, u_shift)
        y, smargin = inverse_cdf_sample(w, u_smp)
        d = len(path) - 1
        out["chosen"][b] = u
        out["accept_len"][b] = d
        out["path"][b, :d + 1] = path
        out["tokens"][b, :d] = [X[b, c] for c in path[1:]]
        out["tokens"][b, d] = y
        out["smp_margin"][b] = smargin
    out["near_tie"] = (out["acc_margin"] < NEAR_TIE) | (out["smp_margin"] < NEAR_TIE)
    return out
