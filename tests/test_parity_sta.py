"""Sliding-tile attention on the GPU (through the C ABI) against the fp64 oracle.

The plan is integer work and must equal the oracle's exactly; outputs are
compared on ragged grids with odd and even windows, the whole-grid window
(dense attention) and the 1x1x1 window, and on sampled cubes of the two
tuned grids the page names, 40 heads each.
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
    o, lse, plan = wf.wf_sta(to_device(q), to_device(k), to_device(v), (wl.T, wl.H, wl.W), window,
                             with_lse=True, with_plan=True)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), plan.cpu().numpy()


def check_heads(wl, q, k, v, o, lse, window, heads, cubes=None):
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)

    def one(bh):
        b, h = bh
        return oracle.sta(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]), synth.bits_to_f64(v[b, h]),
                          tok, wl.T, wl.H, wl.W, window, wl.scale, cubes)
    for bh, (o_ref, l_ref) in zip(heads, pmap(one, heads)):
        m = ~np.isnan(l_ref)
        assert_close(o[bh][m], o_ref[m], f"STA O b{bh[0]} h{bh[1]} ({m.sum()} rows)")
        assert errors(lse[bh][m], l_ref[m])[0] <= LSE_MAX_ABS


@pytest.mark.parametrize("grid,window,B,Hh", [((5, 6, 7), (1, 2, 2), 1, 2), ((13, 10, 23), (3, 3, 3), 1, 1),
                                              ((9, 17, 12), (2, 4, 3), 2, 1), ((4, 4, 4), (1, 1, 1), 1, 1),
                                              ((7, 9, 6), (2, 3, 2), 1, 2), ((1, 1, 1), (1, 1, 1), 1, 1)])
def test_sta_small_grids(wf, grid, window, B, Hh):
    T, H, W = grid
    wl = synth.small_workload("sta_small", B, Hh, T, H, W, 128, structured=True, seed=100 + T, window=window)
    log(f"sta grid={grid} window={window} B={B} Hh={Hh}")
    q, k, v = synth.make_qkv(wl)
    o, lse, plan = gpu_sta(wf, wl, q, k, v, window)
    assert np.array_equal(plan, oracle.sta_plan(T, H, W, window)), "plan differs from the oracle's"
    check_heads(wl, q, k, v, o, lse, window, [(b, h) for b in range(B) for h in range(Hh)])


def test_sta_whole_grid_window_is_dense(wf):
    wl = synth.small_workload("sta_dense", 1, 2, 7, 9, 10, 128, structured=True, seed=110)
    window = (2, 3, 3)
    log("sta whole-grid window vs dense, grid 7x9x10")
    q, k, v = synth.make_qkv(wl)
    o, _, _ = gpu_sta(wf, wl, q, k, v, window)
    od, _ = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v))
    od = od.cpu().numpy()
    for h in range(2):
        ref, _ = oracle.attention(synth.bits_to_f64(q[0, h]), synth.bits_to_f64(k[0, h]),
                                  synth.bits_to_f64(v[0, h]), wl.scale)
        assert_close(o[0, h], ref, f"STA whole grid h{h} vs oracle dense")
        assert_close(o[0, h], od[0, h], f"STA whole grid h{h} vs GPU dense", max_abs=1e-2, mean_abs=1e-3)


@pytest.mark.parametrize("name", ["sta_36x48x48", "sta_18x48x80"])
def test_sta_tuned_grids(wf, name):
    wl = synth.WORKLOADS[name]
    log(f"sta {name} B={wl.B} Hh={wl.Hh} window={wl.window}")
    q, k, v = synth.make_qkv(wl)
    o, lse, plan = gpu_sta(wf, wl, q, k, v, wl.window)
    assert np.array_equal(plan, oracle.sta_plan(wl.T, wl.H, wl.W, wl.window))
    assert np.isfinite(o).all()
    C = plan.shape[0]
    cubes = sorted(set([0, 1, C // 2, C - 2, C - 1] + np.random.default_rng(6).choice(C, 10, replace=False).tolist()))
    check_heads(wl, q, k, v, o, lse, wl.window, [(0, 0), (0, 27)], cubes)


def test_sta_error_paths(wf):
    wl = synth.small_workload("sta_err", 1, 1, 5, 6, 7, 128, seed=111)
    q, k, v = synth.make_qkv(wl)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    with pytest.raises(wf.WfError) as e:
        wf.wf_sta(qd, kd, vd, (5, 6, 7), (3, 1, 1))       # 2 cubes along t
    assert e.value.status == 1
    import torch
    with pytest.raises(wf.WfError) as e:
        wf.wf_sta(qd, kd, vd, (5, 6, 7), (1, 1, 1), workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 3
