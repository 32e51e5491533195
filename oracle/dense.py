"""Dense bidirectional multi-head self-attention, the plain definition in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Anatomy of Wan2.2's 53.6x speedup", section "Why video attention becomes
the bottleneck": dense self-attention compares every query token with every
key token of the 30x52x21 grid; a flash-style kernel never materialises the
score matrix but still performs every query-key and probability-value
product.  The Wan2.1 blog (bafh001.com), section 4.2, calls it without a
causal mask.  So, per (batch, head):

    S = scale * Q K^T          (scale = 1/sqrt(D) unless given)
    P = row-wise softmax(S)    (over all keys, no mask)
    O = P V
    lse_i = log sum_j exp(S_ij)

The softmax is evaluated with the row maximum subtracted first; that is the
same function (a common shift cancels) and cannot overflow.  Section "Fixed-
max softmax is a numerical contract" of the first page explains why a
constant taken from one tile instead of the row maximum is unsafe.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              rows: Optional[Sequence[int]] = None, chunk: int = 1024):
    """Attention of query rows ``rows`` (all when None) over every key.

    q [N, D], k [M, D], v [M, Dv] float64.  Returns (o [R, Dv], lse [R]).
    Rows are processed ``chunk`` at a time so the R x M score block stays small.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    kt = np.ascontiguousarray(k.T)
    for s0 in range(0, rows.size, chunk):
        r = rows[s0:s0 + chunk]
        s = (q[r] @ kt) * scale                  # [R, M] scores
        m = s.max(axis=1)                        # row maximum
        e = np.exp(s - m[:, None])               # unnormalised probabilities
        l = e.sum(axis=1)                        # row sums
        o[s0:s0 + r.size] = (e @ v) / l[:, None]
        lse[s0:s0 + r.size] = m + np.log(l)
    return o, lse


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    rows: Optional[Sequence[int]] = None):
    """attention() for every (b, h) of [B, Hh, N, D] tensors.

    Returns (o [B, Hh, R, Dv], lse [B, Hh, R]).
    """
    B, Hh = q.shape[:2]
    R = q.shape[2] if rows is None else len(rows)
    o = np.empty((B, Hh, R, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hh, R), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            o[b, h], lse[b, h] = attention(q[b, h], k[b, h], v[b, h], scale, rows)
    return o, lse
