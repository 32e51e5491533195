"""Helpers shared by the parity tests: device transfer, error statistics, top-k rule."""
from __future__ import annotations

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Parity bar for floating-point outputs (fp32 GPU output vs fp64 oracle, bf16 inputs).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# lse bar, derived from the arithmetic (test_tolerances.py checks the derivation on the CPU):
# the kernels weight V by the bf16-rounded probabilities and normalise by their sum, so O uses
# one consistent set of weights and the natural-log normaliser they report is the log of that
# same sum (plus the reference).  bf16 keeps 8 significant bits, so round to nearest moves each
# p_j by a relative 2^-8 at most, hence the sum as well: the reported lse is within
# ln(1 + 2^-8) = 3.90e-3 of the exact one.  Rows dominated by one key come close to that
# (3.2e-3 on the benchmark's inputs), so no bar near 1e-3 can hold for these weights.  The
# fp32 parts (scores from D bf16 products, worst-case gamma_D bound; exponentials; the running
# sum over 75,600 keys) add under 6e-4 at the shapes tested; the bar is the sum of the two.
LSE_MAX_ABS = math.log1p(2.0 ** -8) + 6e-4


def log(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a crash still says where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    with ThreadPoolExecutor(threads()) as ex:
        return list(ex.map(fn, items))


def to_device(bits: np.ndarray):
    """bf16 bit patterns (uint16) -> bfloat16 CUDA tensor, bit-exact."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def errors(gpu: np.ndarray, ref: np.ndarray) -> tuple:
    d = np.abs(gpu.astype(np.float64) - ref)
    return float(d.max()), float(d.mean())


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    mx, mn = errors(gpu, ref)
    print(f"  {what}: max-abs {mx:.3e} mean-abs {mn:.3e}", flush=True)
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"


def check_coarse_scores(gpu: np.ndarray, ref: np.ndarray, tau: np.ndarray, what: str) -> None:
    """fp32 coarse scores against the fp64 ones, row by row: row c within tau_c / 4, the
    bound oracle.near_tie_tolerance derives for an fp32 evaluation (and the margin the
    top-k rule relies on)."""
    assert gpu.shape == ref.shape
    err = np.abs(gpu.astype(np.float64) - ref).max(axis=1)
    bad = np.nonzero(~(err <= tau / 4))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows beyond tau_c/4, e.g. row {bad[:5]}"


def check_topk_rows(gpu_idx: np.ndarray, scores: np.ndarray, ref_idx: np.ndarray,
                    margin: np.ndarray, tau: np.ndarray) -> int:
    """Top-k parity under the near-tie rule; returns the number of near-tie rows.

    Rows whose oracle margin exceeds tau must match exactly.  A near-tie row
    passes when the GPU's set is a valid top-k within tau: every kept cube
    scores >= S_(k) - tau and every dropped cube <= S_(k+1) + tau.  Every row
    must be strictly ascending and inside [0, C).
    """
    C, k = ref_idx.shape
    assert gpu_idx.shape == (C, k)
    assert ((gpu_idx >= 0) & (gpu_idx < scores.shape[1])).all(), "index out of range"
    if k > 1:
        assert (np.diff(gpu_idx, axis=1) > 0).all(), "row not strictly ascending"
    exact = margin > tau
    bad = np.nonzero(exact & ~(gpu_idx == ref_idx).all(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ with margin > tau, e.g. row {bad[:5]}"
    near = np.nonzero(~exact)[0]
    srt = -np.sort(-scores, axis=1)
    for r in near:
        kth = srt[r, k - 1]
        nxt = srt[r, k] if k < scores.shape[1] else -np.inf
        chosen = np.zeros(scores.shape[1], bool)
        chosen[gpu_idx[r]] = True
        assert scores[r, chosen].min() >= kth - tau[r], f"near-tie row {r}: kept cube below S_k - tau"
        if (~chosen).any():
            assert scores[r, ~chosen].max() <= nxt + tau[r], f"near-tie row {r}: dropped cube above S_k+1 + tau"
    return int(near.size)
