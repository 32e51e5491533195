"""Sliding-tile attention (STA) over 6x8x8 token tiles, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "推理优化" (Inference optimization, WorldFoundry docs), section on
approximate attention, entry "sta": weight-free sliding-tile attention for
the Wan DiT, accepted only on its tuned token grids (36, 48, 48) and
(18, 48, 80); the default grid (31, 22, 40) of the TI2V 121x704x1280 setting
is refused before any GPU work.  The page gives neither the tile nor the
window size.  Readings adopted (and pinned on their own terms in
tests/test_oracle.py):

1. Tiles are 6 x 8 x 8 tokens (t, h, w).  This is the plainest tile that both
   tuned grids divide without remainder (36/6, 48/8, 48/8 and 18/6, 48/8,
   80/8) and that the refused default grid does not (31 and 22), which is
   what the page's accept/refuse rule implies; so there is no padding and
   every tile holds 384 real tokens.  The oracle accepts any grid the tile
   divides; the library accepts the two tuned grids only, as the page says.
2. Tile (tt, th, tw) has id (tt*nh + th)*nw + tw over the tile grid
   nt x nh x nw = T/6 x H/8 x W/8; inside a tile tokens are row-major.
3. A window of (wt, wh, ww) tiles, 1 <= w <= the tile count on that axis, is
   placed around each query tile: on each axis it starts at
   clamp(c - (w - 1) // 2, 0, n - w), i.e. centred where it fits and shifted
   inward at the grid's edge, so every query tile sees exactly wt*wh*ww key
   tiles (an even w has one more tile above than below).
4. Every query token of a tile attends to every token of the window's tiles
   (softmax over exactly those keys, scale * q . k).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .dense import attention

TILE = (6, 8, 8)                              # reading 1
TUNED_GRIDS = ((36, 48, 48), (18, 48, 80))    # the page's accepted token grids


def tile_grid(T: int, H: int, W: int) -> tuple:
    """(nt, nh, nw) tiles of a T x H x W grid; ValueError unless the tile divides it (reading 1)."""
    bt, bh, bw = TILE
    if T < 1 or H < 1 or W < 1 or T % bt or H % bh or W % bw:
        raise ValueError(f"grid {(T, H, W)} is not a whole number of {TILE} tiles")
    return T // bt, H // bh, W // bw


def tile_tokens(T: int, H: int, W: int) -> np.ndarray:
    """tok[tile, i] = grid index (t*H + h)*W + w of the i-th token (row-major) of each tile: [n, 384]."""
    nt, nh, nw = tile_grid(T, H, W)
    bt, bh, bw = TILE
    t, h, w = np.meshgrid(np.arange(bt), np.arange(bh), np.arange(bw), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    out = np.empty((nt * nh * nw, bt * bh * bw), dtype=np.int64)
    for tt in range(nt):
        for th in range(nh):
            for tw in range(nw):
                out[(tt * nh + th) * nw + tw] = ((tt * bt + t) * H + th * bh + h) * W + tw * bw + w
    return out


def window_start(c: int, w: int, n: int) -> int:
    """First tile of a w-wide window around tile coordinate c on an axis of n tiles (reading 3)."""
    return min(max(c - (w - 1) // 2, 0), n - w)


def sta_plan(T: int, H: int, W: int, window: tuple) -> np.ndarray:
    """[tiles, wt*wh*ww] int64: the key tiles of every query tile's window, ascending (reading 3)."""
    nt, nh, nw = tile_grid(T, H, W)
    wt, wh, ww = window
    if not (1 <= wt <= nt and 1 <= wh <= nh and 1 <= ww <= nw):
        raise ValueError(f"window {window} must fit the tile grid {(nt, nh, nw)}")
    plan = np.empty((nt * nh * nw, wt * wh * ww), dtype=np.int64)
    for ct in range(nt):
        for ch in range(nh):
            for cw in range(nw):
                t0, h0, w0 = window_start(ct, wt, nt), window_start(ch, wh, nh), window_start(cw, ww, nw)
                tiles = [((t * nh) + h) * nw + w for t in range(t0, t0 + wt) for h in range(h0, h0 + wh)
                         for w in range(w0, w0 + ww)]
                plan[(ct * nh + ch) * nw + cw] = sorted(tiles)
    return plan


def sta(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: int, H: int, W: int, window: tuple, scale: float,
        tiles: Optional[Sequence[int]] = None):
    """STA output (o [N, Dv], lse [N]) of one head in grid order (reading 4).

    Rows of query tiles outside ``tiles`` stay NaN.
    """
    tok = tile_tokens(T, H, W)
    plan = sta_plan(T, H, W, window)
    N = q.shape[0]
    o = np.full((N, v.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    for c in (range(tok.shape[0]) if tiles is None else tiles):
        qi = tok[c]
        kj = tok[plan[c]].ravel()
        o[qi], lse[qi] = attention(q[qi], k[kj], v[kj], scale)
    return o, lse
