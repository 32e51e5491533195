"""The library's calls captured in a HIP graph and replayed (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream: it allocates
nothing, issues no memset or copy and never synchronises (the opt-in
WF_VALIDATE index check aside).  So a captured sequence of calls must
reproduce the eager results bit for bit on every replay and must read its
inputs when it is replayed, not when it was captured.  Replays are separated
by eager work of the program's own and a synchronisation, and every output is
poisoned before each replay, so a replay that skipped or reordered a kernel
would show.
"""
import numpy as np
import pytest

import synth
from wf_testutil import log, to_device

pytestmark = pytest.mark.gpu

GRID = (9, 10, 11)  # 990 tokens, padded to 12 x 12 x 12: 27 cubes, ragged in every axis
TOPK = 4
STA_GRID = (18, 48, 80)  # sliding-tile attention runs on its tuned grids only (3 x 6 x 10 tiles)
WINDOW = (1, 2, 3)


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def inputs(seed):
    wl = synth.small_workload("graph", 1, 3, *GRID, 128, structured=True, seed=seed, topk=TOPK)
    q, k, v = (to_device(x) for x in synth.make_qkv(wl))
    ws = synth.small_workload("graph_sta", 1, 1, *STA_GRID, 128, structured=True, seed=seed + 50)
    return q, k, v, to_device(synth.make_gate(wl)), tuple(to_device(x) for x in synth.make_qkv(ws))


def buffers(wf, q):
    """Every output and workspace of the path, allocated once."""
    import torch
    B, Hh, N, D = q.shape
    T, H, W = GRID
    C = wf.num_cubes(T, H, W)
    f32 = dict(dtype=torch.float32, device=q.device)
    ws_sta = wf.lib.wf_sta_workspace_bytes(1, 1, *STA_GRID, D, *WINDOW)
    Ns = STA_GRID[0] * STA_GRID[1] * STA_GRID[2]
    return dict(
        o_dense=torch.empty((B, Hh, N, D), **f32), lse_dense=torch.empty((B, Hh, N), **f32),
        q_rot=torch.empty_like(q), k_rot=torch.empty_like(q),
        idx=torch.empty((B, Hh, C, TOPK), dtype=torch.int32, device=q.device),
        scores=torch.empty((B, Hh, C, C), **f32),
        o_fine=torch.empty((B, Hh, N, D), **f32), lse_fine=torch.empty((B, Hh, N), **f32),
        o_gated=torch.empty((B, Hh, N, D), **f32), o_coarse=torch.empty((B, Hh, C, D), **f32),
        o_sta=torch.empty((1, 1, Ns, D), **f32),
        idx_one=torch.empty((B, Hh, C, TOPK), dtype=torch.int32, device=q.device),
        o_one=torch.empty((B, Hh, N, D), **f32), lse_one=torch.empty((B, Hh, N), **f32),
        ws_dense=torch.empty(wf.dense_workspace_bytes(B, Hh, N, D), dtype=torch.uint8, device=q.device),
        ws_vsa=torch.empty(wf.vsa_workspace_bytes(B, Hh, T, H, W, D), dtype=torch.uint8, device=q.device),
        ws_one=torch.empty(wf.vsa_workspace_bytes(B, Hh, T, H, W, D), dtype=torch.uint8, device=q.device),
        ws_sta=torch.empty(ws_sta, dtype=torch.uint8, device=q.device),
    )


OUTPUTS = ("o_dense", "lse_dense", "q_rot", "k_rot", "idx", "scores", "o_fine", "lse_fine", "o_gated",
           "o_coarse", "o_sta", "idx_one", "o_one", "lse_one")


def path(wf, q, k, v, gate, sta_qkv, b):
    """The whole path once: dense, RoPE, VSA coarse (RoPE fused) + fine + gated, STA, VSA in one call."""
    wf.wf_attn_dense(q, k, v, out=b["o_dense"], lse=b["lse_dense"], workspace=b["ws_dense"])
    wf.wf_rope_qk(q, k, GRID, q_out=b["q_rot"], k_out=b["k_rot"])
    wf.wf_vsa_coarse_topk(q, k, v, GRID, TOPK, idx=b["idx"], scores=b["scores"], workspace=b["ws_vsa"],
                          rope_theta=10000.0)
    wf.wf_vsa_fine(b["ws_vsa"], b["idx"], tuple(q.shape), GRID, out=b["o_fine"], lse=b["lse_fine"])
    wf.wf_vsa_fine_gated(b["ws_vsa"], b["idx"], gate, GRID, out=b["o_gated"], o_coarse=b["o_coarse"])
    wf.wf_sta(*sta_qkv, STA_GRID, WINDOW, out=b["o_sta"], lse=None, workspace=b["ws_sta"])
    wf.wf_vsa(q, k, v, GRID, TOPK, idx=b["idx_one"], out=b["o_one"], lse=b["lse_one"], workspace=b["ws_one"])


def poison(b):
    for name in OUTPUTS:
        t = b[name]
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-1)


def eager(wf, q, k, v, gate, sta_qkv):
    import torch
    b = buffers(wf, q)
    poison(b)
    path(wf, q, k, v, gate, sta_qkv, b)
    torch.cuda.synchronize()
    return {name: b[name].clone() for name in OUTPUTS}


def assert_same(got, want, when):
    import torch
    for name in OUTPUTS:
        g, w = got[name], want[name]
        if g.dtype.is_floating_point:
            assert not torch.isnan(w).any(), f"{name}: NaN in the eager result"
        assert torch.equal(g, w), f"{when}: {name} differs from the eager result"


def test_graph_replays_match_eager(wf):
    import torch
    log("graph capture: eager reference")
    q, k, v, gate, sq = inputs(seed=901)
    want = eager(wf, q, k, v, gate, sq)

    log("graph capture: capture the path")
    b = buffers(wf, q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path(wf, q, k, v, gate, sq, b)
    torch.cuda.synchronize()

    x = torch.randn(512, 512, device=q.device)
    for r in range(3):
        log(f"graph capture: replay {r}")
        poison(b)
        y = x @ x  # the program's own work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        assert_same(b, want, f"replay {r}")

    log("graph capture: new input contents, replay")
    q2, k2, v2, gate2, sq2 = inputs(seed=902)
    want2 = eager(wf, q2, k2, v2, gate2, sq2)
    assert not torch.equal(want2["o_dense"], want["o_dense"])
    assert not torch.equal(want2["o_sta"], want["o_sta"])
    for dst, src in ((q, q2), (k, k2), (v, v2), (gate, gate2)) + tuple(zip(sq, sq2)):
        dst.copy_(src)
    poison(b)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert_same(b, want2, "replay on new inputs")
    np.testing.assert_array_equal(b["idx"].cpu().numpy(), want2["idx"].cpu().numpy())
