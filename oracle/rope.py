"""3D rotary position embedding (RoPE) of Q and K on the video token grid, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "推理优化" (Inference optimization, WorldFoundry docs,
openenvision.org), section "Exact or numerically equivalent Wan kernels",
entry fused_rope: a fused 3D RoPE for the Wan DiT whose rotation runs in
fp32 or fp64, and which can take a sequence-parallel rank's offset.  The page
gives no frequencies or axis split, so the following definition is adopted
(the common one for Wan-style 3D RoPE) and every part of it is pinned on its
own terms in tests/test_oracle.py:

1. The head dimension D (even) is cut into three consecutive parts for the
   three grid axes: d_t = D - 4*floor(D/6) dims for t, then
   d_h = d_w = 2*floor(D/6) dims for h and for w (D = 128: 44, 42, 42).
2. Inside an axis part of d_a dims, elements (2i, 2i+1) form pair i, which
   rotates by the angle pos_a * theta**(-2i / d_a), pos_a being the token's
   0-based coordinate on that axis and theta the frequency base (10000).
3. A pair (x0, x1) rotated by phi becomes
   (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi).
4. Q and K are rotated, V is not, and the result is rounded to bf16, round
   to nearest even, since attention consumes bf16 Q and K.  The page's two
   precisions are both defined: "fp64" rotates in fp64 arithmetic; "fp32"
   rounds cos and sin (taken in fp64) to fp32 and then forms
   x0*c - x1*s and x0*s + x1*c with each product and the sum rounded to fp32
   (no fused multiply-add), so the bf16 rounding decision is taken on that
   fp32 value.
"""
from __future__ import annotations

import numpy as np


def axis_split(D: int) -> tuple:
    """(d_t, d_h, d_w) of the head dimension (definition 1)."""
    if D % 2 or D < 6:
        raise ValueError("D must be even and at least 6")
    f = D // 6
    return D - 4 * f, 2 * f, 2 * f


def grid_positions(T: int, H: int, W: int) -> np.ndarray:
    """(t, h, w) integer coordinates of every token in row-major order, [N, 3]."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)


def angles(pos: np.ndarray, D: int, theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of every pair (definition 2): [N, D/2] for positions [N, 3]."""
    cols = []
    for axis, d_a in enumerate(axis_split(D)):
        freq = theta ** (-2.0 * np.arange(d_a // 2) / d_a)
        cols.append(pos[:, axis:axis + 1].astype(np.float64) * freq[None, :])
    return np.concatenate(cols, axis=1)


def rotate(x: np.ndarray, phi: np.ndarray, precision: str = "fp64") -> np.ndarray:
    """Rotate the pairs (x[:, 2i], x[:, 2i+1]) of x [N, D] by phi [N, D/2] (definitions 3, 4).

    Returns float64; with precision "fp32" every value is an fp32 result.
    """
    if precision == "fp64":
        x0, x1 = x[:, 0::2], x[:, 1::2]
        c, s = np.cos(phi), np.sin(phi)
    elif precision == "fp32":
        x0, x1 = x[:, 0::2].astype(np.float32), x[:, 1::2].astype(np.float32)
        c, s = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
    else:
        raise ValueError("precision is 'fp64' or 'fp32'")
    out = np.empty(x.shape, dtype=np.float64)
    out[:, 0::2] = x0 * c - x1 * s      # float32 operands: each step rounds to fp32
    out[:, 1::2] = x0 * s + x1 * c
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value (8 significant bits), ties to even.

    Written for the normal bf16 range, which is all the rotated Q and K reach:
    x = m * 2**e with 0.5 <= |m| < 1 (frexp), and m * 256 is rounded to an
    integer, halves to even (numpy's rint).
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def rope(x: np.ndarray, T: int, H: int, W: int, theta: float = 10000.0,
         precision: str = "fp64") -> np.ndarray:
    """x [N, D] (N = T*H*W, row-major (t, h, w)) rotated, not rounded to bf16."""
    if x.shape[0] != T * H * W:
        raise ValueError("x must hold the T*H*W tokens of the grid")
    return rotate(x, angles(grid_positions(T, H, W), x.shape[1], theta), precision)


def rope_bf16(x: np.ndarray, T: int, H: int, W: int, theta: float = 10000.0,
              precision: str = "fp64") -> np.ndarray:
    """What attention consumes: the rotation of x rounded to bf16 (definition 4)."""
    return round_bf16(rope(x, T, H, W, theta, precision))
