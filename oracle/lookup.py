"""Prompt-lookup drafting: the plain definition, one sequence at a time.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's CPU
baseline, never by the product path.

"Speculative decoding explained", section "Variants without a separate draft model": prompt
lookup needs no draft model; it scans the prompt and the conversation history for phrases
that appear again in the response and offers what followed them as draft candidates.

Reading (the page gives no procedure): for n from max_ngram down to min_ngram, the last n
tokens of the history are the phrase; its earliest earlier occurrence, one that starts at
i with i + n < len (so at least one token follows it), is the match; the drafts are the up
to k tokens that follow the match, h[i+n .. min(i+n+k, len)), padded with -1.  The first n
(largest first) that matches decides; no match for any n gives no drafts.  A length
outside [0, cap] is not a history at all and drafts nothing.
"""
from __future__ import annotations

import numpy as np


def lookup_drafts(history, seq_len, min_ngram: int, max_ngram: int, k: int):
    """history int [B, cap]; seq_len int [B].  Returns (drafts [B, k] int64, -1 padded,
    count [B] int64)."""
    history = np.asarray(history)
    B = history.shape[0]
    drafts = np.full((B, k), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    for b in range(B):
        length = int(seq_len[b])
        if length < 0 or length > history.shape[1]:
            continue
        h = [int(t) for t in history[b, :length]]
        for n in range(max_ngram, min_ngram - 1, -1):
            if n < 1 or n >= length:
                continue
            phrase = h[length - n:]
            match = -1
            for i in range(0, length - n):
                if h[i:i + n] == phrase:
                    match = i
                    break
            if match < 0:
                continue
            follow = h[match + n:min(match + n + k, length)]
            drafts[b, :len(follow)] = follow
            count[b] = len(follow)
            break
    return drafts, count
