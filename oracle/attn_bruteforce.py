"""Brute-force softmax attention split over KV chunks -- TEST INFRASTRUCTURE ONLY.

This is what produces the partials the merge consumes: each DCP rank attends
over its own slice of the KV cache and returns (out_r, lse_r); a rank whose
slice is empty returns the neutral pair (0, -inf) (sglang PR #33926 report,
实现拆解 item 3).  Merging the per-slice partials must reproduce attention over
the whole KV, which is the property that pins the oracle's combine: the pages
call the merge an exact LSE-weighted reduction (vLLM PR #41160 report, 功能与动机).

KV ownership follows the round-robin rule of the sglang PR #33926 report
(关键源码片段, TestDcpDecodeLayout): token t belongs to rank t mod n.  A
contiguous split is provided too.  Plain numpy, fp64.
"""
from __future__ import annotations

import numpy as np


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Single-query attention per head.

    q [H, dk], K [L, dk], V [L, D] (fp64).  Returns (out [H, D], lse [H]) with
    lse the natural-log sum of exp(scores).  L == 0 returns the neutral pair.
    """
    H = q.shape[0]
    D = V.shape[1]
    L = K.shape[0]
    if L == 0:
        return np.zeros((H, D)), np.full((H,), -np.inf)
    s = (q @ K.T) * scale                      # [H, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    den = p.sum(axis=1)
    out = (p @ V) / den[:, None]
    lse = m[:, 0] + np.log(den)
    return out, lse


def round_robin_owner(L: int, n: int) -> np.ndarray:
    """Rank that owns each KV token: t mod n."""
    return np.arange(L) % n


def contiguous_owner(L: int, n: int) -> np.ndarray:
    """Rank that owns each KV token when the KV is cut into n near-equal blocks."""
    return (np.arange(L) * n) // max(L, 1)


def split_partials(q, K, V, scale, owner: np.ndarray, n: int):
    """Per-rank partials (out [n, H, D], lse [n, H]) over the tokens each owns."""
    outs, lses = [], []
    for r in range(n):
        idx = np.nonzero(owner == r)[0]
        o, l = attention(q, K[idx], V[idx], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
