"""Video Sparse Attention (VSA) on a 3D token grid, step by step in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "VSA
selects cubes".  The grid is padded to multiples of 4 and split into 4x4x4
cubes of 64 tokens (21x30x52 becomes 24x32x52 = 39,936 tokens and
6x8x13 = 624 cubes).  The coarse stage averages each cube's query and key
vectors into one representative vector, runs cheap cube-level attention and
ranks candidate key cubes; the fine stage runs full token-level attention of
each query cube over only its top-ranked key and value cubes.  At 87.5%
sparsity 78 of the 624 cubes are kept.  Section "Roofline analysis set the
3.35 ms target" fixes the cost conventions: 624 query cubes x 40 heads =
24,960 output tiles, about 3.35 TFLOP with padded query tokens left out, and
about 64 GB of streamed K/V.

Readings taken where the page is silent (each one is tested):

1. Cube numbering is row-major over the cube grid, c = (ct*nh + ch)*nw + cw,
   and a token's slot inside its cube is row-major too,
   slot = (t%4*4 + h%4)*4 + w%4.  This only names cubes and slots.
2. The cube mean is taken over the cube's real (unpadded) tokens only; a
   cube never holds zero real tokens because padding stops below the next
   multiple of 4.
3. Ranking uses the raw coarse scores scale * Qbar_c . Kbar_c'; a row
   softmax is monotone, so it selects the same set.
4. No cube is forced into the selection (no forced diagonal).
5. Ties go to the larger score first, then the smaller key-cube index; the
   selected indices are reported in ascending order.
6. Padded key slots are masked out of the fine softmax, and padded query
   slots produce no output.
7. The gate of the merge comes from learned weights, so it is an input here:
   the caller supplies it (``gated``); the plain VSA output is the fine
   stage's.
8. The coarse branch's output for query cube c is its cube-level attention
   over all C key cubes: the row softmax of the same scaled cube-mean scores,
   times the key cubes' mean values (real tokens, as in reading 2).  The
   section says the merge keeps the fine result whole and adds a learned
   share of the coarse branch, so each real token of cube c receives
   O = O_fine + g * O_coarse[c], elementwise, with g of the output's shape
   [N, D] per head.  The log-sum-exp reported is the fine stage's.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .dense import attention

CUBE = 4  # cube edge, in tokens, along t, h and w


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def geometry(T: int, H: int, W: int) -> dict:
    """Padded grid and cube grid of a real T x H x W token grid."""
    nt, nh, nw = _ceil_div(T, CUBE), _ceil_div(H, CUBE), _ceil_div(W, CUBE)
    C = nt * nh * nw
    return dict(T=T, H=H, W=W, N=T * H * W, Tp=CUBE * nt, Hp=CUBE * nh, Wp=CUBE * nw,
                nt=nt, nh=nh, nw=nw, C=C, Np=C * CUBE ** 3)


def cube_layout(T: int, H: int, W: int) -> np.ndarray:
    """tok[c, slot] = grid index (t*H + h)*W + w of the token in that cube slot, -1 if padded.

    Shape [C, 64] int64.  Every padded-grid position is visited once.
    """
    g = geometry(T, H, W)
    tp, hp, wp = np.meshgrid(np.arange(g["Tp"]), np.arange(g["Hp"]), np.arange(g["Wp"]),
                             indexing="ij")
    tp, hp, wp = tp.ravel(), hp.ravel(), wp.ravel()
    cube = ((tp // CUBE) * g["nh"] + hp // CUBE) * g["nw"] + wp // CUBE
    slot = ((tp % CUBE) * CUBE + hp % CUBE) * CUBE + wp % CUBE
    real = (tp < T) & (hp < H) & (wp < W)
    tok = np.full((g["C"], CUBE ** 3), -1, dtype=np.int64)
    tok[cube[real], slot[real]] = (tp[real] * H + hp[real]) * W + wp[real]
    return tok


def pool(x: np.ndarray, tok: np.ndarray) -> np.ndarray:
    """Cube means of x [N, D] over each cube's real tokens (reading 2): [C, D]."""
    valid = tok >= 0
    gathered = np.where(valid[:, :, None], x[np.maximum(tok, 0)], 0.0)
    return gathered.sum(axis=1) / valid.sum(axis=1)[:, None]


def coarse_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """Cube-level scores S_c[c, c'] = scale * Qbar_c . Kbar_c' (reading 3): [C, C]."""
    return (qbar @ kbar.T) * scale


def select_topk(scores: np.ndarray, k: int):
    """Top-k key cubes of every row (reading 5).

    Returns (idx [C, k] int64 ascending, margin [C]) where margin is the
    k-th best score minus the (k+1)-th (inf when k equals the cube count).
    """
    C, Ck = scores.shape
    if not 1 <= k <= Ck:
        raise ValueError(f"top-k {k} outside [1, {Ck}]")
    # a stable sort of the negated scores: descending score, equal scores by ascending index
    order = np.argsort(-scores, axis=1, kind="stable")
    idx = np.sort(order[:, :k], axis=1)
    margin = np.full(C, np.inf)
    if k < Ck:
        kth = np.take_along_axis(scores, order[:, k - 1:k], axis=1)[:, 0]
        nxt = np.take_along_axis(scores, order[:, k:k + 1], axis=1)[:, 0]
        margin = kth - nxt
    return idx, margin


def near_tie_tolerance(q: np.ndarray, k: np.ndarray, tok: np.ndarray, scale: float) -> np.ndarray:
    """Per-row tolerance tau_c = 2^-14 * scale * max_c' sum_d A_c,d B_c',d.

    A and B are the cube means of |q| and |k| over real tokens.  An fp32
    evaluation of the cube means (sums of at most 64 terms, then a divide)
    and of the D-term coarse dot product (D <= 256), in any summation
    order, lands within tau/4 of the exact score, so a row whose top-k
    margin exceeds tau has exactly one correct selection in fp32 too.
    """
    A, B = pool(np.abs(q), tok), pool(np.abs(k), tok)
    return (A @ B.T).max(axis=1) * scale * 2.0 ** -14


def fine(q: np.ndarray, k: np.ndarray, v: np.ndarray, tok: np.ndarray, idx: np.ndarray,
         scale: float, cubes: Optional[Sequence[int]] = None):
    """Fine stage (readings 6): each query cube attends over its selected cubes' real keys.

    q, k [N, D], v [N, Dv] in grid order; idx [C, k].  Returns (o [N, Dv],
    lse [N]) in grid order; rows of query cubes outside ``cubes`` stay NaN.
    """
    N = q.shape[0]
    o = np.full((N, v.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    for c in (range(tok.shape[0]) if cubes is None else cubes):
        qi = tok[c][tok[c] >= 0]
        sel = tok[np.asarray(idx[c])]
        kj = sel[sel >= 0]
        o[qi], lse[qi] = attention(q[qi], k[kj], v[kj], scale)
    return o, lse


def vsa(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: int, H: int, W: int, topk: int,
        scale: float, cubes: Optional[Sequence[int]] = None, idx: Optional[np.ndarray] = None):
    """Whole VSA pass for one (batch, head): pool, score, select, fine attention.

    With ``idx`` given, the selection step is skipped and that plan is used.
    Returns a dict with qbar, kbar, scores, idx, margin, tau, o, lse.
    """
    tok = cube_layout(T, H, W)
    qbar, kbar = pool(q, tok), pool(k, tok)
    scores = coarse_scores(qbar, kbar, scale)
    sel, margin = select_topk(scores, topk)
    plan = sel if idx is None else np.asarray(idx)
    o, lse = fine(q, k, v, tok, plan, scale, cubes)
    return dict(qbar=qbar, kbar=kbar, scores=scores, idx=sel, margin=margin,
                tau=near_tie_tolerance(q, k, tok, scale), o=o, lse=lse)


def coarse_output(qbar: np.ndarray, kbar: np.ndarray, vbar: np.ndarray, scale: float) -> np.ndarray:
    """Coarse-branch output per query cube (reading 8): softmax over all key cubes of
    scale * Qbar_c . Kbar_c', times Vbar: [C, D]."""
    s = coarse_scores(qbar, kbar, scale)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ vbar


def gated(q: np.ndarray, k: np.ndarray, v: np.ndarray, tok: np.ndarray, idx: np.ndarray, scale: float,
          gate: np.ndarray, cubes: Optional[Sequence[int]] = None):
    """Fine output plus gate * coarse output of each token's query cube (readings 7, 8).

    gate: [N, D].  Returns (o, lse) like ``fine``: rows of query cubes outside
    ``cubes`` are NaN, and lse is the fine stage's.
    """
    o, lse = fine(q, k, v, tok, idx, scale, cubes)
    oc = coarse_output(pool(q, tok), pool(k, tok), pool(v, tok), scale)
    cube_of = np.full(q.shape[0], -1, dtype=np.int64)
    rows, slots = np.nonzero(tok >= 0)
    cube_of[tok[rows, slots]] = rows
    return o + gate * oc[cube_of], lse


def flops_fine(N: int, topk: int, D: int, heads: int, batch: int = 1) -> float:
    """Fine-stage FLOPs in the page's convention: 4 * N * (64 k) * D per head.

    Padded query tokens are left out; every slot of a selected key cube counts.
    """
    return 4.0 * N * (CUBE ** 3 * topk) * D * heads * batch


def kv_stream_bytes(C: int, topk: int, D: int, heads: int, batch: int = 1,
                    elem_bytes: int = 2) -> float:
    """K and V bytes streamed when every output tile reads its k cubes once."""
    return float(batch * heads * C * CUBE ** 3 * topk * D * 2 * elem_bytes)
