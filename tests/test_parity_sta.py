"""Sliding-tile attention on the GPU (through the C ABI) against the fp64 oracle.

STA runs on the two tuned token grids only (the library refuses the rest with
WF_ERR_UNSUPPORTED, as the inference-optimization page says it must).  The
tile plan is integer work and must equal the oracle's exactly; outputs are
compared on every row of the heads checked: odd, even, single-tile and
edge-hugging windows on both grids, the whole-grid window (dense attention),
and the benchmark's 40-head calls (every row written; two heads compared
whole).  Outputs are poisoned before every call.
"""
import numpy as np
import pytest

import oracle
import synth
from wf_testutil import LSE_MAX_ABS, assert_close, errors, log, pmap, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def gpu_sta(wf, wl, q, k, v, window):
    import torch
    T, H, W = wl.T, wl.H, wl.W
    o = torch.full((wl.B, wl.Hh, wl.N, wl.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.B, wl.Hh, wl.N), float("nan"), dtype=torch.float32, device="cuda")
    o, lse, plan = wf.wf_sta(to_device(q), to_device(k), to_device(v), (T, H, W), window, out=o, lse=lse,
                             with_plan=True)
    torch.cuda.synchronize()
    o, lse, plan = o.cpu().numpy(), lse.cpu().numpy(), plan.cpu().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "output rows never written"
    return o, lse, plan


def check_heads(wl, q, k, v, o, lse, window, heads, tiles=None):
    def one(bh):
        b, h = bh
        return oracle.sta(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]), synth.bits_to_f64(v[b, h]),
                          wl.T, wl.H, wl.W, window, wl.scale, tiles)
    for bh, (o_ref, l_ref) in zip(heads, pmap(one, heads)):
        m = ~np.isnan(l_ref)
        assert_close(o[bh][m], o_ref[m], f"STA O b{bh[0]} h{bh[1]} ({m.sum()} rows)")
        assert errors(lse[bh][m], l_ref[m])[0] <= LSE_MAX_ABS


@pytest.mark.parametrize("grid,window,B,Hh", [((36, 48, 48), (3, 3, 3), 1, 2), ((36, 48, 48), (2, 4, 1), 2, 1),
                                              ((36, 48, 48), (1, 1, 1), 1, 1), ((18, 48, 80), (3, 3, 3), 1, 1),
                                              ((18, 48, 80), (2, 1, 4), 1, 2), ((18, 48, 80), (1, 6, 2), 1, 1)])
def test_sta_tuned_grids_all_rows(wf, grid, window, B, Hh):
    T, H, W = grid
    wl = synth.small_workload("sta", B, Hh, T, H, W, 128, structured=True, seed=100 + sum(window), window=window)
    log(f"sta grid={grid} window={window} B={B} Hh={Hh}")
    q, k, v = synth.make_qkv(wl)
    o, lse, plan = gpu_sta(wf, wl, q, k, v, window)
    assert np.array_equal(plan, oracle.sta_plan(T, H, W, window)), "plan differs from the oracle's"
    check_heads(wl, q, k, v, o, lse, window, [(b, h) for b in range(B) for h in range(Hh)])


def test_sta_whole_grid_window_is_dense(wf):
    wl = synth.small_workload("sta_dense", 1, 1, 18, 48, 80, 128, structured=True, seed=110)
    window = (3, 6, 10)
    log("sta whole-grid window vs dense, grid 18x48x80")
    q, k, v = synth.make_qkv(wl)
    o, _, _ = gpu_sta(wf, wl, q, k, v, window)
    od, _ = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v))
    od = od.cpu().numpy()
    ref, _ = oracle.attention(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]), synth.bits_to_f64(v[0, 0]),
                              wl.scale)
    assert_close(o[0, 0], ref, "STA whole grid vs oracle dense")
    assert_close(o[0, 0], od[0, 0], "STA whole grid vs GPU dense", max_abs=1e-2, mean_abs=1e-3)


@pytest.mark.parametrize("name", ["sta_36x48x48", "sta_18x48x80"])
def test_sta_benchmark_calls(wf, name):
    wl = synth.WORKLOADS[name]
    log(f"sta {name} B={wl.B} Hh={wl.Hh} window={wl.window}")
    q, k, v = synth.make_qkv(wl)
    o, lse, plan = gpu_sta(wf, wl, q, k, v, wl.window)
    assert np.array_equal(plan, oracle.sta_plan(wl.T, wl.H, wl.W, wl.window))
    check_heads(wl, q, k, v, o, lse, wl.window, [(0, 0), (0, 27)])


def test_sta_error_paths(wf):
    import torch
    for grid in ((31, 22, 40), (5, 6, 7), (36, 48, 40), (18, 48, 48)):
        wl = synth.small_workload("sta_err", 1, 1, *grid, 128, seed=111)
        q, k, v = synth.make_qkv(wl)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        with pytest.raises(wf.WfError) as e:       # not a tuned grid: refused before any GPU work
            wf.wf_sta(qd, kd, vd, grid, (1, 1, 1))
        assert e.value.status == 2
        assert wf.lib.wf_sta_workspace_bytes(1, 1, *grid, 128, 1, 1, 1) == 0
    wl = synth.small_workload("sta_err", 1, 1, 18, 48, 80, 128, seed=112)
    q, k, v = synth.make_qkv(wl)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    for window in ((4, 1, 1), (1, 7, 1), (1, 1, 11), (0, 1, 1)):
        with pytest.raises(wf.WfError) as e:
            wf.wf_sta(qd, kd, vd, (18, 48, 80), window)
        assert e.value.status == 1
    with pytest.raises(wf.WfError) as e:
        wf.wf_sta(qd, kd, vd, (18, 48, 80), (1, 1, 1), workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 3
