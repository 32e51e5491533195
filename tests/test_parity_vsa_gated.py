"""VSA's gated merge on the GPU (through the C ABI) against the fp64 oracle.

The coarse-branch output (cube-level softmax over all key cubes times the
cube means of V) is compared for every query cube, the merged output
O = O_fine + gate * O_coarse[cube] for every real token (small grids) or
sampled cubes (480p and the 4,096-cube limit), and gate = 0 must reproduce
the fine stage's output bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from wf_testutil import LSE_MAX_ABS, assert_close, errors, log, pmap, to_device

pytestmark = pytest.mark.gpu

# The coarse product runs with split bf16 operands and fp32 sums; its error is
# near fp32's, far inside the attention bar (the comparison below uses it).
COARSE_MAX_ABS = 1e-3
COARSE_MEAN_ABS = 1e-4


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def gpu_gated(wf, wl, q, k, v, gate):
    import torch
    grid = (wl.T, wl.H, wl.W)
    qd, kd, vd, gd = to_device(q), to_device(k), to_device(v), to_device(gate)
    idx, _, ws = wf.wf_vsa_coarse_topk(qd, kd, vd, grid, wl.topk)
    o, lse, oc = wf.wf_vsa_fine_gated(ws, idx, gd, grid, with_lse=True, with_coarse=True)
    of, lf = wf.wf_vsa_fine(ws, idx, tuple(qd.shape), grid, with_lse=True)
    torch.cuda.synchronize()
    return dict(idx=idx.cpu().numpy(), o=o.cpu().numpy(), lse=lse.cpu().numpy(),
                oc=oc.cpu().numpy(), of=of.cpu().numpy(), lf=lf.cpu().numpy(), ws=ws, idx_dev=idx)


def ref_coarse(wl, q, k, v, tok, bh):
    b, h = bh
    qf, kf, vf = (synth.bits_to_f64(x[b, h]) for x in (q, k, v))
    return oracle.coarse_output(oracle.pool(qf, tok), oracle.pool(kf, tok), oracle.pool(vf, tok), wl.scale)


def check_heads(wl, q, k, v, gate, g, tok, heads, cubes=None):
    """O_coarse for every cube; gated O and lse against the oracle on the GPU's own plan."""
    def one(bh):
        b, h = bh
        oc = ref_coarse(wl, q, k, v, tok, bh)
        o, lse = oracle.gated(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]),
                              synth.bits_to_f64(v[b, h]), tok, g["idx"][bh], wl.scale,
                              synth.bits_to_f64(gate[b, h]), cubes)
        return oc, o, lse
    for bh, (oc, o_ref, l_ref) in zip(heads, pmap(one, heads)):
        assert_close(g["oc"][bh], oc, f"O_coarse b{bh[0]} h{bh[1]}", COARSE_MAX_ABS, COARSE_MEAN_ABS)
        m = ~np.isnan(l_ref)
        assert_close(g["o"][bh][m], o_ref[m], f"gated O b{bh[0]} h{bh[1]} ({m.sum()} rows)")
        assert errors(g["lse"][bh][m], l_ref[m])[0] <= LSE_MAX_ABS
        # lse is the fine stage's, bit for bit
        assert np.array_equal(g["lse"][bh][m], g["lf"][bh][m])


@pytest.mark.parametrize("grid,topk,B,Hh", [((5, 6, 7), 3, 1, 2), ((9, 10, 11), 5, 2, 1),
                                            ((4, 4, 4), 1, 1, 1), ((1, 1, 1), 1, 1, 1),
                                            ((13, 6, 21), 17, 1, 2), ((3, 17, 9), 2, 1, 1), ((10, 9, 14), 6, 1, 1)])
def test_vsa_gated_small_grids(wf, grid, topk, B, Hh):
    T, H, W = grid
    wl = synth.small_workload("vsa_gated", B, Hh, T, H, W, 128, structured=True,
                              seed=500 + T * 10 + topk, topk=topk)
    log(f"vsa gated grid={grid} topk={topk} B={B} Hh={Hh}")
    q, k, v = synth.make_qkv(wl)
    gate = synth.make_gate(wl)
    g = gpu_gated(wf, wl, q, k, v, gate)
    tok = oracle.cube_layout(T, H, W)
    check_heads(wl, q, k, v, gate, g, tok, [(b, h) for b in range(B) for h in range(Hh)])


def test_vsa_gate_zero_is_fine_output(wf):
    wl = synth.small_workload("vsa_gate0", 1, 3, 9, 10, 11, 128, structured=True, seed=510, topk=4)
    log("vsa gate=0 vs fine grid 9x10x11")
    q, k, v = synth.make_qkv(wl)
    g = gpu_gated(wf, wl, q, k, v, np.zeros_like(q))
    assert np.array_equal(g["o"], g["of"]), "gate = 0 must reproduce the fine output exactly"
    assert np.array_equal(g["lse"], g["lf"])


def test_vsa_gated_iid_inputs(wf):
    """Unstructured inputs: the coarse softmax is spread over many cubes, not peaked."""
    wl = synth.small_workload("vsa_gated_iid", 1, 2, 12, 16, 20, 128, structured=False, seed=511, topk=6)
    log("vsa gated iid grid 12x16x20")
    q, k, v = synth.make_qkv(wl)
    gate = synth.make_gate(wl)
    g = gpu_gated(wf, wl, q, k, v, gate)
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    check_heads(wl, q, k, v, gate, g, tok, [(0, 0), (0, 1)])


def test_vsa_gated_480p(wf):
    """480p, 40 heads, top-32: O_coarse of every head in full, gated O on sampled cubes."""
    wl = synth.WORKLOADS["vsa_480p"]
    log(f"vsa gated {wl.name} B={wl.B} Hh={wl.Hh} topk={wl.topk}")
    q, k, v = synth.make_qkv(wl)
    gate = synth.make_gate(wl)
    g = gpu_gated(wf, wl, q, k, v, gate)
    assert np.isfinite(g["o"]).all()
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    heads = [(0, h) for h in range(wl.Hh)]
    refs = pmap(lambda bh: ref_coarse(wl, q, k, v, tok, bh), heads)
    for bh, oc in zip(heads, refs):
        assert_close(g["oc"][bh], oc, f"O_coarse h{bh[1]}", COARSE_MAX_ABS, COARSE_MEAN_ABS)
    cubes = sorted(set([0, 12, 13, 311, 622, 623] +
                       np.random.default_rng(7).choice(tok.shape[0], 12, replace=False).tolist()))
    check_heads(wl, q, k, v, gate, g, tok, [(0, 2), (0, 29)], cubes)


def test_vsa_gated_max_cubes(wf):
    """4,096 cubes (the widest top-k path and the largest coarse product), top-64."""
    wl = synth.small_workload("vsa_gated_max", 1, 1, 61, 62, 63, 128, structured=True, seed=41, topk=64)
    log(f"vsa gated max cubes grid {wl.T}x{wl.H}x{wl.W}")
    q, k, v = synth.make_qkv(wl)
    gate = synth.make_gate(wl)
    g = gpu_gated(wf, wl, q, k, v, gate)
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    cubes = sorted(set([0, 15, 255, 2048, 4095] +
                       np.random.default_rng(41).choice(4096, 7, replace=False).tolist()))
    check_heads(wl, q, k, v, gate, g, tok, [(0, 0)], cubes)


def test_vsa_gated_error_paths(wf):
    import torch
    wl = synth.small_workload("vsa_gated_err", 1, 1, 5, 6, 7, 128, seed=512, topk=2)
    q, k, v = synth.make_qkv(wl)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    idx, _, ws = wf.wf_vsa_coarse_topk(qd, kd, vd, (5, 6, 7), 2)
    with pytest.raises(ValueError):
        wf.wf_vsa_fine_gated(ws, idx, qd.float(), (5, 6, 7))
    with pytest.raises(wf.WfError) as e:
        wf.wf_vsa_fine_gated(ws[:64], idx, qd, (5, 6, 7))
    assert e.value.status == 3
    torch.cuda.synchronize()


def test_vsa_gated_after_fused_rope(wf):
    """The gated call on the workspace of the RoPE-fused coarse stage equals the oracle's gated merge on
    the oracle-rotated Q and K (the whole VSA chain with both additions)."""
    import torch
    wl = synth.small_workload("vsa_gated_rope", 1, 2, 9, 10, 11, 128, structured=True, seed=513, topk=4)
    log("vsa gated after fused rope, grid 9x10x11")
    q, k, v = synth.make_qkv(wl)
    gate = synth.make_gate(wl)
    grid = (wl.T, wl.H, wl.W)
    idx, _, ws = wf.wf_vsa_coarse_topk(to_device(q), to_device(k), to_device(v), grid, wl.topk,
                                       rope_theta=10000.0, rope_precision=64)
    o, lse, oc = wf.wf_vsa_fine_gated(ws, idx, to_device(gate), grid, with_lse=True, with_coarse=True)
    torch.cuda.synchronize()
    g = dict(idx=idx.cpu().numpy(), o=o.cpu().numpy(), lse=lse.cpu().numpy(), oc=oc.cpu().numpy())
    tok = oracle.cube_layout(wl.T, wl.H, wl.W)
    rot = lambda x: synth.bf16_bits(np.stack([np.stack([
        oracle.rope_bf16(synth.bits_to_f64(x[b, h]), wl.T, wl.H, wl.W, 10000.0, "fp64").astype(np.float32)
        for h in range(wl.Hh)]) for b in range(wl.B)]))
    qr, kr = rot(q), rot(k)
    for h in range(wl.Hh):
        qf, kf, vf = synth.bits_to_f64(qr[0, h]), synth.bits_to_f64(kr[0, h]), synth.bits_to_f64(v[0, h])
        oc_ref = oracle.coarse_output(oracle.pool(qf, tok), oracle.pool(kf, tok), oracle.pool(vf, tok), wl.scale)
        assert_close(g["oc"][0, h], oc_ref, f"O_coarse after rope h{h}", COARSE_MAX_ABS, COARSE_MEAN_ABS)
        o_ref, l_ref = oracle.gated(qf, kf, vf, tok, g["idx"][0, h], wl.scale, synth.bits_to_f64(gate[0, h]))
        assert_close(g["o"][0, h], o_ref, f"gated O after rope h{h}")
        assert errors(g["lse"][0, h], l_ref)[0] <= LSE_MAX_ABS


def test_vsa_gated_validates_plans(wf, monkeypatch):
    import torch
    wl = synth.small_workload("vsa_gated_val", 1, 1, 9, 10, 11, 128, structured=True, seed=514, topk=3)
    log("vsa gated with WF_VALIDATE, bad plan")
    q, k, v = synth.make_qkv(wl)
    grid = (wl.T, wl.H, wl.W)
    idx, _, ws = wf.wf_vsa_coarse_topk(to_device(q), to_device(k), to_device(v), grid, wl.topk)
    bad = idx.clone()
    bad[0, 0, 4, 2] = bad[0, 0, 4, 1]          # a repeated cube: not strictly ascending
    monkeypatch.setenv("WF_VALIDATE", "1")
    wf.wf_vsa_fine_gated(ws, idx, to_device(q), grid)   # the coarse stage's own plan passes
    with pytest.raises(wf.WfError) as e:
        wf.wf_vsa_fine_gated(ws, bad, to_device(q), grid)
    assert e.value.status == 4
    monkeypatch.delenv("WF_VALIDATE")
    torch.cuda.synchronize()
