"""VSA on the GPU (through the C ABI) against the fp64 oracle.

Checks the selected key-cube indices (exactly, under the near-tie rule), the
fine-stage output (the GPU's whole pipeline, and the fine stage alone on the
GPU's own plan), the closed forms (Q = 0 ties, top-k = all cubes equals
dense attention) and the error paths.  Outputs are poisoned before every call.
The 480p and 720p workloads are checked whole in test_parity_full.py.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from wf_testutil import (LSE_MAX_ABS, assert_close, check_coarse_scores, check_topk_rows, errors, log,
                         pmap, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def gpu_vsa(wf, wl, q, k, v, topk=None):
    """Both stages on outputs poisoned first (NaN, indices -1): every entry must be written."""
    import torch
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    topk = topk or wl.topk
    C = wf.num_cubes(wl.T, wl.H, wl.W)
    idx = torch.full((wl.B, wl.Hh, C, topk), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((wl.B, wl.Hh, C, C), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full(tuple(qd.shape), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(tuple(qd.shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    idx, scores, ws = wf.wf_vsa_coarse_topk(qd, kd, vd, (wl.T, wl.H, wl.W), topk, with_scores=True,
                                            idx=idx, scores=sc)
    o, lse = wf.wf_vsa_fine(ws, idx, tuple(qd.shape), (wl.T, wl.H, wl.W), out=o, lse=lse)
    torch.cuda.synchronize()
    assert not (idx < 0).any().item() and not torch.isnan(scores).any().item()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    return dict(idx=idx.cpu().numpy(), scores=scores.cpu().numpy(), o=o.cpu().numpy(),
                lse=lse.cpu().numpy(), ws=ws, idx_dev=idx)


def coarse_ref(wl, q, k, heads, topk):
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)

    def one(bh):
        b, h = bh
        qf, kf = synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h])
        qb, kb = oracle.pool(qf, tok), oracle.pool(kf, tok)
        sc = oracle.coarse_scores(qb, kb, wl.scale)
        idx, margin = oracle.select_topk(sc, topk)
        return dict(scores=sc, idx=idx, margin=margin,
                    tau=oracle.near_tie_tolerance(qf, kf, tok, wl.scale))
    return dict(zip(heads, pmap(one, heads))), tok


def check_scores_and_idx(g, ref, heads):
    near = 0
    for bh in heads:
        r = ref[bh]
        # fp32 scores within the tolerance the top-k rule assumes, row by row
        check_coarse_scores(g["scores"][bh], r["scores"], r["tau"], f"scores b{bh[0]} h{bh[1]}")
        near += check_topk_rows(g["idx"][bh], r["scores"], r["idx"], r["margin"], r["tau"])
    print(f"  near-tie rows: {near} of {len(heads) * g['idx'].shape[2]}", flush=True)
    return near


def check_fine(wl, q, k, v, g, tok, heads, cubes=None, topk=None):
    def one(bh):
        b, h = bh
        return oracle.fine(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]),
                           synth.bits_to_f64(v[b, h]), tok, g["idx"][bh], wl.scale, cubes)
    res = pmap(one, heads)
    for bh, (o_ref, l_ref) in zip(heads, res):
        m = ~np.isnan(l_ref)
        assert_close(g["o"][bh][m], o_ref[m], f"fine O b{bh[0]} h{bh[1]} ({m.sum()} rows)")
        assert errors(g["lse"][bh][m], l_ref[m])[0] <= LSE_MAX_ABS


@pytest.mark.parametrize("grid,topk,B,Hh", [((5, 6, 7), 1, 1, 2), ((5, 6, 7), 3, 2, 1),
                                            ((5, 6, 7), 8, 1, 1), ((9, 10, 11), 5, 1, 2),
                                            ((4, 4, 4), 1, 1, 1), ((1, 1, 1), 1, 1, 1),
                                            ((13, 6, 21), 17, 1, 2), ((6, 11, 14), 7, 1, 2)])
def test_vsa_small_grids_all_outputs(wf, grid, topk, B, Hh):
    T, H, W = grid
    wl = synth.small_workload("vsa_small", B, Hh, T, H, W, 128, structured=True, seed=T * 100 + topk,
                              topk=topk)
    log(f"vsa small grid={grid} topk={topk} B={B} Hh={Hh}")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    heads = [(b, h) for b in range(B) for h in range(Hh)]
    ref, tok = coarse_ref(wl, q, k, heads, topk)
    check_scores_and_idx(g, ref, heads)
    check_fine(wl, q, k, v, g, tok, heads)


def test_vsa_all_cubes_equals_dense(wf):
    wl = synth.small_workload("vsa_all", 1, 2, 7, 9, 10, 128, structured=True, seed=21)
    C = wf.num_cubes(wl.T, wl.H, wl.W)
    log(f"vsa topk=C={C} vs dense, grid 7x9x10")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v, topk=C)
    assert (g["idx"] == np.arange(C)).all()
    import torch
    od, _ = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v))
    od = od.cpu().numpy()
    for h in range(2):
        ref, _ = oracle.attention(synth.bits_to_f64(q[0, h]), synth.bits_to_f64(k[0, h]),
                                  synth.bits_to_f64(v[0, h]), wl.scale)
        assert_close(g["o"][0, h], ref, f"VSA(k=C) h{h} vs oracle dense")
        assert_close(g["o"][0, h], od[0, h], f"VSA(k=C) h{h} vs GPU dense", max_abs=1e-2, mean_abs=1e-3)


def test_vsa_zero_queries_tie_rule(wf):
    wl = synth.small_workload("vsa_q0", 1, 1, 8, 12, 9, 128, structured=True, seed=22, topk=4)
    log("vsa Q=0 ties grid 8x12x9 topk=4")
    q, k, v = synth.make_qkv(wl)
    q[:] = 0
    g = gpu_vsa(wf, wl, q, k, v)
    C = g["idx"].shape[2]
    assert (g["idx"][0, 0] == np.arange(4)).all(), "equal scores must resolve to the smallest cubes"
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    sel = tok[:4].ravel()
    expect = synth.bits_to_f64(v[0, 0])[sel[sel >= 0]].mean(axis=0)
    assert_close(g["o"][0, 0], np.broadcast_to(expect, g["o"][0, 0].shape), "Q=0 O", max_abs=2e-3,
                 mean_abs=5e-4)
    assert C == 2 * 3 * 3


def test_vsa_480p_k78(wf):
    """The review's operating point: 78 of 624 cubes kept."""
    wl = synth.WORKLOADS["vsa_480p_k78"]
    log(f"vsa {wl.name} B={wl.B} Hh={wl.Hh} topk={wl.topk} (all heads idx)")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    heads = [(0, h) for h in range(wl.Hh)]
    ref, tok = coarse_ref(wl, q, k, heads, wl.topk)
    check_scores_and_idx(g, ref, heads)
    cubes = sorted(np.random.default_rng(78).choice(tok.shape[0], 24, replace=False).tolist() + [0, 623])
    check_fine(wl, q, k, v, g, tok, [(0, 5), (0, 33)], cubes)


def test_vsa_max_cubes(wf):
    """The largest supported plan: 4,096 cubes (16 x 16 x 16, every axis padded), top-64.

    Exercises the widest top-k path (more than 2,048 cubes per row) and the
    fine stage's 32-bit offsets at the cube limit.
    """
    wl = synth.small_workload("vsa_max", 1, 1, 61, 62, 63, 128, structured=True, seed=40, topk=64)
    log(f"vsa max cubes grid {wl.T}x{wl.H}x{wl.W} N={wl.N} topk={wl.topk}")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    heads = [(0, 0)]
    ref, tok = coarse_ref(wl, q, k, heads, wl.topk)
    assert tok.shape[0] == 4096
    check_scores_and_idx(g, ref, heads)
    assert np.isfinite(g["o"]).all()
    cubes = sorted(set([0, 15, 16, 255, 256, 2047, 2048, 4080, 4095] +
                       np.random.default_rng(40).choice(4096, 11, replace=False).tolist()))
    check_fine(wl, q, k, v, g, tok, heads, cubes)


def test_vsa_fine_caller_plan_and_validation(wf, monkeypatch):
    """A caller-supplied plan runs as given; with WF_VALIDATE=1 a bad plan is refused."""
    import torch
    wl = synth.small_workload("vsa_plan", 1, 2, 9, 10, 11, 128, structured=True, seed=23, topk=3)
    log("vsa caller plan + validation grid 9x10x11")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    C = g["idx"].shape[2]
    rng = np.random.default_rng(0)
    plan = np.sort(np.stack([np.stack([rng.choice(C, 3, replace=False) for _ in range(C)])
                             for _ in range(2)])[None], axis=-1).astype(np.int32)
    plan_d = torch.from_numpy(plan).cuda()
    shape = (1, 2, wl.N, 128)
    monkeypatch.setenv("WF_VALIDATE", "1")
    o, lse = wf.wf_vsa_fine(g["ws"], plan_d, shape, (wl.T, wl.H, wl.W), with_lse=True)
    o = o.cpu().numpy()
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    for h in range(2):
        ref, _ = oracle.fine(synth.bits_to_f64(q[0, h]), synth.bits_to_f64(k[0, h]),
                             synth.bits_to_f64(v[0, h]), tok, plan[0, h], wl.scale)
        assert_close(o[0, h], ref, f"caller plan h{h}")
    for bad in ("dup", "range", "order"):
        p = plan.copy()
        if bad == "dup":
            p[0, 1, 5, 1] = p[0, 1, 5, 0]
        elif bad == "range":
            p[0, 0, 2, 2] = C
        else:
            p[0, 0, 7] = p[0, 0, 7][::-1]
        with pytest.raises(wf.WfError) as e:
            wf.wf_vsa_fine(g["ws"], torch.from_numpy(p).cuda(), shape, (wl.T, wl.H, wl.W))
        assert e.value.status == 4
    monkeypatch.delenv("WF_VALIDATE")


@pytest.mark.parametrize("plan", [[6], [4], [2], [18], [6, 9], [0, 6], [6, 9, 10], [2, 9, 10], [18, 19, 21],
                                  [0, 1, 6], [6, 7, 8], [17, 25, 26], [18, 6], [19, 6, 21], [6, 20, 9]])
def test_vsa_fine_edge_cube_plans(wf, plan):
    """The same caller plan for every query cube of a 9x10x11 grid (27 cubes, 19 of them edge cubes):
    each kind of edge cube (padded along t, h or w, or several) first, in the middle and last,
    and k = 1, 2, 3, so that the masked key slots of the first tile, of later tiles and of the
    last tile are all exercised; every output row is compared with the oracle.  Cubes 18..26 (the
    last layer along t, one frame deep) have their second half all padding; the last three plans
    put them before whole cubes, which an ascending plan never does, to exercise every transition
    of the fine stage's half-tile path (the result does not depend on the order of the plan)."""
    import torch
    wl = synth.small_workload("vsa_edge_plans", 1, 2, 9, 10, 11, 128, structured=True, seed=23, topk=3)
    log(f"vsa fine, plan {plan} for every query cube, grid 9x10x11")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    C = g["idx"].shape[2]
    pl = np.broadcast_to(np.array(plan, np.int32), (1, 2, C, len(plan))).copy()
    o = torch.full((1, 2, wl.N, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((1, 2, wl.N), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = wf.wf_vsa_fine(g["ws"], torch.from_numpy(pl).cuda(), (1, 2, wl.N, 128), (wl.T, wl.H, wl.W),
                            out=o, lse=lse)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    for h in range(2):
        ref, lref = oracle.fine(synth.bits_to_f64(q[0, h]), synth.bits_to_f64(k[0, h]),
                                synth.bits_to_f64(v[0, h]), tok, pl[0, h], wl.scale)
        assert_close(o[0, h], ref, f"plan {plan} head {h}")
        assert np.abs(lse[0, h] - lref).max() <= LSE_MAX_ABS, f"plan {plan} head {h}: lse"


@pytest.mark.parametrize("grid,topk,B,Hh", [((5, 6, 7), 3, 1, 2), ((9, 10, 11), 5, 2, 1), ((1, 1, 1), 1, 1, 1),
                                            ((13, 6, 21), 17, 1, 2), ((21, 30, 52), 32, 1, 3),
                                            ((9, 17, 29), 64, 1, 2), ((21, 30, 52), 78, 1, 1),
                                            ((10, 9, 14), 12, 1, 2)])
def test_vsa_one_call_equals_two_calls(wf, grid, topk, B, Hh):
    """wf_vsa (no cube-ordered copies of Q, K and V; the fine stage reads them from the token grid,
    V through transpose reads) gives the plan, O and lse of wf_vsa_coarse_topk + wf_vsa_fine bit for
    bit, and O matches the oracle's fine stage on that plan, up to top-78.  T % 4 of 1 and 2 puts
    cubes in the last layer whose second half (slots 32..63) is padding, which the fine stage
    treats apart (no work for that half of the query rows, half the MFMAs for such a key cube)."""
    import torch
    T, H, W = grid
    wl = synth.small_workload("vsa_one_call", B, Hh, T, H, W, 128, structured=True, seed=T * 7 + topk, topk=topk)
    log(f"vsa one call grid={grid} topk={topk} B={B} Hh={Hh}")
    q, k, v = synth.make_qkv(wl)
    g = gpu_vsa(wf, wl, q, k, v)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    C = g["idx"].shape[2]
    idx = torch.full((B, Hh, C, topk), -1, dtype=torch.int32, device="cuda")
    o = torch.full(tuple(qd.shape), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(tuple(qd.shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    o, lse, idx = wf.wf_vsa(qd, kd, vd, (T, H, W), topk, idx=idx, out=o, lse=lse)
    o, lse, idx = o.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    assert (idx == g["idx"]).all(), "plan differs from the two-call path"
    assert np.array_equal(o.view(np.uint32), g["o"].view(np.uint32)), "O differs from the two-call path"
    assert np.array_equal(lse.view(np.uint32), g["lse"].view(np.uint32)), "lse differs from the two-call path"
    # with a gate: the gated merge of wf_vsa_fine_gated on the two-call workspace, bit for bit
    gate = to_device(synth.make_gate(wl))
    og2, _, oc2 = wf.wf_vsa_fine_gated(g["ws"], g["idx_dev"], gate, (T, H, W), with_coarse=True)
    oc1 = torch.full((B, Hh, C, 128), float("nan"), dtype=torch.float32, device="cuda")
    og1 = torch.full(tuple(qd.shape), float("nan"), dtype=torch.float32, device="cuda")
    og1, _, _ = wf.wf_vsa(qd, kd, vd, (T, H, W), topk, out=og1, gate=gate, o_coarse=oc1)
    assert torch.equal(og1.view(torch.int32), og2.view(torch.int32)), "gated O differs from the two-call path"
    assert torch.equal(oc1.view(torch.int32), oc2.view(torch.int32)), "O_coarse differs from the two-call path"
    tok = oracle.cube_layout(T, H, W)
    for b in range(B):
        for h in range(min(Hh, 2)):
            ref, lref = oracle.fine(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]),
                                    synth.bits_to_f64(v[b, h]), tok, idx[b, h], wl.scale,
                                    None if T * H * W < 8192 else list(range(0, C, 7)))
            m = ~np.isnan(lref)
            assert_close(o[b, h][m], ref[m], f"one call b{b} h{h}")
            assert errors(lse[b, h][m], lref[m])[0] <= LSE_MAX_ABS


def test_vsa_error_paths(wf):
    import torch
    wl = synth.small_workload("vsa_err", 1, 1, 5, 6, 7, 128, seed=24)
    q, k, v = synth.make_qkv(wl)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    for topk in (0, 9):
        with pytest.raises(wf.WfError) as e:
            wf.wf_vsa_coarse_topk(qd, kd, vd, (5, 6, 7), topk)
        assert e.value.status == 1
    with pytest.raises(wf.WfError) as e:
        wf.wf_vsa_coarse_topk(qd, kd, vd, (5, 6, 7), 2, workspace=torch.empty(64, dtype=torch.uint8,
                                                                                device="cuda"))
    assert e.value.status == 3
    q64 = to_device(q[..., :64].copy())
    with pytest.raises(wf.WfError) as e:
        wf.wf_vsa_coarse_topk(q64, q64, q64, (5, 6, 7), 2)
    assert e.value.status == 2
