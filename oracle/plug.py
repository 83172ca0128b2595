"""Token plug after verification: the plain definition, one sequence at a time.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's CPU
baseline, never by the product path.

"Accelerating Sonar through speculation", section "MTP schedule for one token": once the
target's input tokens are shifted, the next tokens are plugged into their positions on the
GPU, so no GPU-to-CPU read of the accepted lengths is needed before the next step.  The
operation is an append: sequence b's emitted tokens (out_tokens[b, 0..n], n its accepted
length) go to the end of its token history, which grows by n + 1 (up to its capacity), and
the last emitted token is the next step's input.
"""
from __future__ import annotations

import numpy as np

OK, TRUNCATED, INVALID = 0, 1, 2


def plug_tokens(out_tokens, accept_len, seq_len, history):
    """Returns (seq_len', history', next_token, status) without modifying the inputs.

    out_tokens int [B, W]; accept_len int [B]; seq_len int [B]; history int [B, cap].
    next_token is -1 where nothing was appended (status INVALID)."""
    out_tokens = np.asarray(out_tokens)
    B, W = out_tokens.shape
    hist = np.array(history, copy=True)
    cap = hist.shape[1]
    lens = np.array(seq_len, copy=True)
    nxt = np.full(B, -1, dtype=np.int64)
    status = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(accept_len[b])
        start = int(lens[b])
        if not (0 <= n < W) or not (0 <= start <= cap):
            status[b] = INVALID
            continue
        for i in range(n + 1):
            if start + i < cap:
                hist[b, start + i] = out_tokens[b, i]
        nxt[b] = out_tokens[b, n]
        end = start + n + 1
        status[b] = TRUNCATED if end > cap else OK
        lens[b] = min(end, cap)
    return lens, hist, nxt, status
