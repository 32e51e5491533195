"""Softmax reference policies on the GPU against the fp64 oracle.

"Anatomy of Wan2.2's 53.6x speedup", section "Fixed-max softmax is a numerical
contract": a reduction constant taken from the first selected tile keeps the
softmax exact while later scores stay in range, and overflows the
exponential when a later score is much larger.  Checked here:

* on ordinary inputs the guarded default, the running-max online softmax
  and the unguarded first-tile constant all meet the parity bar;
* on an adversarial input whose later keys score ~181 (natural log units)
  above the first tile's, the unguarded constant turns the affected rows into
  inf / NaN, while the guarded default and the running max stay exact;
* just inside the range (later scores ~45 above), even the unguarded
  constant is exact.
"""
import numpy as np
import pytest

import oracle
import synth
from wf_testutil import LSE_MAX_ABS, assert_close, errors, log, to_device

pytestmark = pytest.mark.gpu

MODES = {0: "guarded", 1: "running max", 2: "fixed first tile"}


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_dense_modes_ordinary_inputs(wf, mode):
    wl = synth.small_workload("dense_modes", 1, 2, 5, 9, 11, 128, structured=True, seed=90)
    log(f"dense softmax {MODES[mode]} grid 5x9x11")
    q, k, v = synth.make_qkv(wl)
    o, lse = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v), with_lse=True, softmax_mode=mode)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for h in range(2):
        ref, lref = oracle.attention(synth.bits_to_f64(q[0, h]), synth.bits_to_f64(k[0, h]),
                                     synth.bits_to_f64(v[0, h]), wl.scale)
        assert_close(o[0, h], ref, f"dense {MODES[mode]} h{h}")
        assert errors(lse[0, h], lref)[0] <= LSE_MAX_ABS


def adversarial_dense(gain):
    """1 head, N = 256, D = 128: keys 0..63 score 0, keys 128..191 score gain * 5.66 (natural log)."""
    N, D = 256, 128
    r = np.random.default_rng(91)
    q = np.full((N, D), 0.5, np.float32)
    k = r.normal(scale=0.05, size=(N, D)).astype(np.float32)
    k[:64] = 0.0
    k[128:192] = gain
    v = r.normal(size=(N, D)).astype(np.float32)
    return bf16(q)[None, None], bf16(k)[None, None], bf16(v)[None, None]


def test_dense_overflow_case(wf):
    q, k, v = adversarial_dense(32.0)        # later scores ~181 above the first tile's
    scale = 1 / np.sqrt(128)
    ref, lref = oracle.attention(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]),
                                 synth.bits_to_f64(v[0, 0]), scale)
    assert np.isfinite(ref).all()
    log("dense overflow case, three policies")
    out = {}
    for mode in (0, 1, 2):
        o, lse = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v), with_lse=True, softmax_mode=mode)
        out[mode] = (o.cpu().numpy()[0, 0], lse.cpu().numpy()[0, 0])
    bad = ~np.isfinite(out[2][0])
    print(f"  fixed first tile: {bad.sum()} of {bad.size} outputs non-finite", flush=True)
    assert bad.all(axis=1).all(), "every row's later keys overflow the first tile's constant"
    for mode in (0, 1):
        assert_close(out[mode][0], ref, f"dense overflow case, {MODES[mode]}")
        assert errors(out[mode][1], lref)[0] <= LSE_MAX_ABS


def test_dense_near_overflow_is_exact_for_all(wf):
    q, k, v = adversarial_dense(8.0)         # later scores ~45 above: exp stays finite
    scale = 1 / np.sqrt(128)
    ref, _ = oracle.attention(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]),
                              synth.bits_to_f64(v[0, 0]), scale)
    log("dense near-overflow case, three policies")
    for mode in (0, 1, 2):
        o, _ = wf.wf_attn_dense(to_device(q), to_device(k), to_device(v), softmax_mode=mode)
        assert_close(o.cpu().numpy()[0, 0], ref, f"dense near overflow, {MODES[mode]}")


def vsa_fine_modes(wf, wl, q, k, v, plan):
    import torch
    grid = (wl.T, wl.H, wl.W)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    _, _, ws = wf.wf_vsa_coarse_topk(qd, kd, vd, grid, plan.shape[-1])
    plan_d = torch.from_numpy(plan).cuda()
    res = {}
    for mode in (0, 1, 2):
        o, lse = wf.wf_vsa_fine(ws, plan_d, tuple(q.shape), grid, with_lse=True, softmax_mode=mode)
        res[mode] = (o.cpu().numpy()[0, 0], lse.cpu().numpy()[0, 0])
    return res


def test_vsa_modes_ordinary_and_overflow(wf):
    """8x8x8 grid (8 cubes), plan [0, 5, 7] for every query cube; cube 5's keys made large."""
    wl = synth.small_workload("vsa_modes", 1, 1, 8, 8, 8, 128, structured=True, seed=92, topk=3)
    q, k, v = synth.make_qkv(wl)
    tok = oracle.cube_layout(8, 8, 8)
    plan = np.tile(np.array([0, 5, 7], np.int32), (8, 1))[None, None]
    log("vsa fine, three policies, ordinary inputs")
    res = vsa_fine_modes(wf, wl, q, k, v, plan)
    ref, lref = oracle.fine(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]), synth.bits_to_f64(v[0, 0]),
                            tok, plan[0, 0], wl.scale)
    for mode in (0, 1, 2):
        assert_close(res[mode][0], ref, f"vsa ordinary, {MODES[mode]}")
    # adversarial: queries 0.5, keys of cube 0 zero, keys of cube 5 at 32 (scores ~181 natural)
    q[:] = bf16(0.5)
    kk = synth.bits_to_f64(k[0, 0]) * 0.05
    kk[tok[0]] = 0.0
    kk[tok[5]] = 32.0
    k[0, 0] = bf16(kk)
    log("vsa fine, three policies, overflow case")
    res = vsa_fine_modes(wf, wl, q, k, v, plan)
    ref, lref = oracle.fine(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]), synth.bits_to_f64(v[0, 0]),
                            tok, plan[0, 0], wl.scale)
    assert np.isfinite(ref).all()
    bad = ~np.isfinite(res[2][0])
    print(f"  fixed first tile: {bad.sum()} of {bad.size} outputs non-finite", flush=True)
    assert bad.all(axis=1).all()
    for mode in (0, 1):
        assert_close(res[mode][0], ref, f"vsa overflow case, {MODES[mode]}")
        assert errors(res[mode][1], lref)[0] <= LSE_MAX_ABS


def test_softmax_mode_rejected(wf):
    wl = synth.small_workload("modes_err", 1, 1, 2, 3, 4, 128, seed=93)
    q, k, v = synth.make_qkv(wl)
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_dense(to_device(q), to_device(k), to_device(v), softmax_mode=5)
    assert e.value.status == 1
