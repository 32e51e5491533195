"""Sliding-tile attention (STA) over the 4x4x4 cube layout, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "推理优化" (Inference optimization, WorldFoundry docs), section on
approximate attention, entry "sta": weight-free sliding-tile attention for
the Wan DiT, accepted only on its tuned token grids (36, 48, 48) and
(18, 48, 80).  The page gives neither tile nor window sizes, so the
following definition is adopted and pinned on its own terms in
tests/test_oracle.py:

1. Tiles are VSA's 4x4x4 cubes of the padded grid (oracle.vsa.cube_layout),
   so padded slots exist and are masked exactly as in VSA's fine stage.
2. A window of (wt, wh, ww) cubes, 1 <= w <= the cube count on that axis, is
   placed around each query cube c: on each axis it starts at
   clamp(c_axis - (w - 1) // 2, 0, n_axis - w), i.e. centred where it fits and
   shifted inward at the grid's edge, so every query cube sees exactly
   wt * wh * ww key cubes (an even w has one more cube above than below).
3. Every real query token of cube c attends to every real key token of the
   window's cubes: the VSA fine stage with that plan (listed ascending).
"""
from __future__ import annotations

import numpy as np

from .vsa import fine, geometry


def window_start(c: int, w: int, n: int) -> int:
    """First cube of a w-wide window around cube coordinate c on an axis of n cubes."""
    return min(max(c - (w - 1) // 2, 0), n - w)


def sta_plan(T: int, H: int, W: int, window: tuple) -> np.ndarray:
    """[C, wt*wh*ww] int64: the key cubes of every query cube's window, ascending (definition 2)."""
    g = geometry(T, H, W)
    nt, nh, nw = g["nt"], g["nh"], g["nw"]
    wt, wh, ww = window
    if not (1 <= wt <= nt and 1 <= wh <= nh and 1 <= ww <= nw):
        raise ValueError(f"window {window} must fit the cube grid {(nt, nh, nw)}")
    plan = np.empty((nt * nh * nw, wt * wh * ww), dtype=np.int64)
    for ct in range(nt):
        for ch in range(nh):
            for cw in range(nw):
                t0, h0, w0 = window_start(ct, wt, nt), window_start(ch, wh, nh), window_start(cw, ww, nw)
                cubes = [((t * nh) + h) * nw + w for t in range(t0, t0 + wt) for h in range(h0, h0 + wh)
                         for w in range(w0, w0 + ww)]
                plan[(ct * nh + ch) * nw + cw] = sorted(cubes)
    return plan


def sta(q: np.ndarray, k: np.ndarray, v: np.ndarray, tok: np.ndarray, T: int, H: int, W: int,
        window: tuple, scale: float, cubes=None):
    """STA output (o [N, D], lse [N]) of one head (definition 3); rows outside `cubes` are NaN."""
    return fine(q, k, v, tok, sta_plan(T, H, W, window), scale, cubes)
