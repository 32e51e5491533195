"""Seeded synthetic Q/K/V for video-DiT self-attention workloads.

This module is the only code shared by the fp64 oracle side and the HIP side:
it draws inputs and nothing else.  It holds no attention arithmetic (no
products, softmax, pooling, cube mapping or selection).

Recipe (the pages print no tensors, so these inputs stand in for the
real-shape Wan2.2 480p tensors that "Anatomy of Wan2.2's 53.6x speedup"
(zharfai.com), section "Fixed-max softmax is a numerical contract", says
were published separately and are not available here):

* positions p = (t/(T-1), h/(H-1), w/(W-1)) over the real (unpadded) grid,
  tokens in row-major (t, h, w) order;
* a random-Fourier-feature field phi_j(p) = sqrt(2) cos(omega_j . p + beta_j),
  j < D, with omega_j ~ N(0, l^-2 I_3), beta_j ~ U[0, 2 pi), l = 0.15, so
  that E[phi_j^2] = 1 and nearby positions get strongly correlated features;
* X = bf16_RNE(z + 2 phi(p_n)) with z ~ N(0, 1) iid per element, one field
  shared by Q, K, V, every head and every batch entry.  The "iid" workloads
  use z alone.

Every (tensor, b, h) slice has its own PCG64 stream seeded by
SeedSequence([seed, tensor_id, b, h]) so any slice regenerates on its own.

The gate of VSA's gated merge (a learned share of the coarse branch, an
input here) is G = bf16_RNE(u), u ~ U[0, 1) iid per element, from the stream
of tensor id 3.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Iterable, Optional

import numpy as np

LENGTH_SCALE = 0.15
FIELD_GAIN = 2.0
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "gate": 3}
_FIELD_STREAM = 1000  # SeedSequence entropy suffix for the shared field


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, input recipe and (for VSA) top-k."""

    name: str
    B: int
    Hh: int
    T: int
    H: int
    W: int
    D: int
    structured: bool  # True: N(0,1) + 2*phi ; False: N(0,1) iid
    seed: int
    topk: Optional[int] = None
    window: Optional[tuple] = None  # sliding-tile attention window, in cubes
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


# The five measured configurations, plus dense attention on the 720p tensors and VSA at the
# review's 78-of-624 operating point.
WORKLOADS = {
    "dense_512_iid": Workload("dense_512_iid", 1, 2, 8, 8, 8, 64, False, 1,
                              note="dense MHA, 8x8x8 grid, d64, iid N(0,1)"),
    "dense_480p_12h": Workload("dense_480p_12h", 1, 12, 21, 30, 52, 128, True, 2,
                               note="dense MHA, 480p grid 21x30x52, 12 heads"),
    "dense_480p_cfg": Workload("dense_480p_cfg", 2, 40, 21, 30, 52, 128, True, 3,
                               note="dense MHA, 480p grid, CFG pair x 40 heads"),
    "vsa_480p": Workload("vsa_480p", 1, 40, 21, 30, 52, 128, True, 4, topk=32,
                         note="VSA, 480p grid padded to 24x32x52, 624 cubes, top-32"),
    "vsa_720p": Workload("vsa_720p", 2, 40, 21, 45, 80, 128, True, 5, topk=64,
                         note="VSA, 720p grid padded to 24x48x80, 1440 cubes, top-64"),
    # dense attention on the same 720p tensors (same seed) for comparison with VSA
    "dense_720p_cfg": Workload("dense_720p_cfg", 2, 40, 21, 45, 80, 128, True, 5,
                               note="dense MHA, 720p grid 21x45x80, CFG pair x 40 heads"),
    # the page's operating point: 78 of 624 cubes (87.5% sparsity)
    "vsa_480p_k78": Workload("vsa_480p_k78", 1, 40, 21, 30, 52, 128, True, 4, topk=78,
                             note="VSA, 480p grid, 624 cubes, top-78 (the review's 87.5% sparsity)"),
    # sliding-tile attention on its two tuned token grids, 3x3x3-tile windows of 6x8x8-token tiles
    "sta_36x48x48": Workload("sta_36x48x48", 1, 40, 36, 48, 48, 128, True, 6, window=(3, 3, 3),
                             note="STA, grid 36x48x48 (6x6x6 tiles of 6x8x8), window 3x3x3 tiles"),
    "sta_18x48x80": Workload("sta_18x48x80", 1, 40, 18, 48, 80, 128, True, 7, window=(3, 3, 3),
                             note="STA, grid 18x48x80 (3x6x10 tiles of 6x8x8), window 3x3x3 tiles"),
}


def positions(T: int, H: int, W: int) -> np.ndarray:
    """Normalised (t, h, w) coordinates of the real grid, [N, 3] float64, row-major."""
    def axis(n):
        return np.zeros(1) if n == 1 else np.arange(n, dtype=np.float64) / (n - 1)
    t, h, w = np.meshgrid(axis(T), axis(H), axis(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)


def fourier_field(T: int, H: int, W: int, D: int, seed: int) -> np.ndarray:
    """phi(p_n) for every real token, [N, D] float32 (computed in float64)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _FIELD_STREAM])))
    omega = rng.standard_normal((D, 3)) / LENGTH_SCALE
    beta = rng.uniform(0.0, 2.0 * np.pi, size=D)
    p = positions(T, H, W)
    return (np.sqrt(2.0) * np.cos(p @ omega.T + beta)).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bits_to_f32(bits).astype(np.float64)


def _slice(wl: Workload, tensor: str, b: int, h: int, phi: Optional[np.ndarray]) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([wl.seed, TENSOR_IDS[tensor], b, h])))
    z = rng.standard_normal((wl.N, wl.D), dtype=np.float32)
    if phi is not None:
        z += np.float32(FIELD_GAIN) * phi
    return bf16_bits(z)


def field_for(wl: Workload) -> Optional[np.ndarray]:
    return fourier_field(wl.T, wl.H, wl.W, wl.D, wl.seed) if wl.structured else None


def make_slice(wl: Workload, tensor: str, b: int, h: int,
               phi: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits [N, D] of one (b, h) slice of tensor 'q', 'k' or 'v'."""
    if phi is None and wl.structured:
        phi = field_for(wl)
    return _slice(wl, tensor, b, h, phi)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_tensor(wl: Workload, tensor: str, out: Optional[np.ndarray] = None,
                phi: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits [B, Hh, N, D] of a whole tensor, slices drawn in parallel."""
    if phi is None and wl.structured:
        phi = field_for(wl)
    if out is None:
        out = np.empty((wl.B, wl.Hh, wl.N, wl.D), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, wl.Hh)
        out[b, h] = _slice(wl, tensor, b, h, phi)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(wl.B * wl.Hh)))
    return out


def make_gate_slice(wl: Workload, b: int, h: int) -> np.ndarray:
    """bf16 bits [N, D] of one (b, h) slice of the gate, U[0, 1) per element."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([wl.seed, TENSOR_IDS["gate"], b, h])))
    return bf16_bits(rng.random((wl.N, wl.D), dtype=np.float32))


def make_gate(wl: Workload) -> np.ndarray:
    """bf16 bits [B, Hh, N, D] of the whole gate."""
    out = np.empty((wl.B, wl.Hh, wl.N, wl.D), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, wl.Hh)
        out[b, h] = make_gate_slice(wl, b, h)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(wl.B * wl.Hh)))
    return out


def make_qkv(wl: Workload) -> tuple:
    """(q, k, v) bf16 bits, each [B, Hh, N, D]."""
    phi = field_for(wl)
    return tuple(make_tensor(wl, t, phi=phi) for t in ("q", "k", "v"))


def make_qkv_heads(wl: Workload, heads: Iterable[tuple]) -> dict:
    """{(b, h): (q, k, v)} bf16 bits [N, D] for selected heads only."""
    phi = field_for(wl)
    return {(b, h): tuple(_slice(wl, t, b, h, phi) for t in ("q", "k", "v"))
            for (b, h) in heads}


def small_workload(name: str, B: int, Hh: int, T: int, H: int, W: int, D: int,
                   structured: bool = True, seed: int = 11, topk: Optional[int] = None,
                   window: Optional[tuple] = None) -> Workload:
    """An ad-hoc workload for tests (same recipe, any shape)."""
    return Workload(name, B, Hh, T, H, W, D, structured, seed, topk, window)
