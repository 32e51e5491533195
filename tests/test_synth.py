"""The seeded input generator: determinism, bf16 rounding, field statistics."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.normal(size=100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, -1e-40], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_regenerate_independently():
    wl = synth.small_workload("t", 2, 3, 3, 4, 5, 16, structured=True, seed=7)
    q, k, v = synth.make_qkv(wl)
    assert q.shape == (2, 3, 60, 16) and q.dtype == np.uint16
    assert np.array_equal(synth.make_slice(wl, "k", 1, 2), k[1, 2])
    heads = synth.make_qkv_heads(wl, [(0, 1)])
    assert np.array_equal(heads[(0, 1)][2], v[0, 1])
    assert not np.array_equal(q[0, 0], k[0, 0])
    q2, _, _ = synth.make_qkv(wl)
    assert np.array_equal(q, q2)


def test_positions_and_field():
    p = synth.positions(3, 1, 5)
    assert p.shape == (15, 3)
    np.testing.assert_allclose(p[-1], [1.0, 0.0, 1.0])
    np.testing.assert_allclose(p[1], [0.0, 0.0, 0.25])
    phi = synth.fourier_field(21, 30, 52, 128, 4)
    assert phi.shape == (32760, 128)
    assert abs(float((phi.astype(np.float64) ** 2).mean()) - 1.0) < 0.05
    # neighbouring tokens are strongly correlated, far ones are not
    a, b, far = phi[0].astype(np.float64), phi[1].astype(np.float64), phi[-1].astype(np.float64)
    assert a @ b / 128 > 0.9
    assert abs(a @ far / 128) < 0.3


def test_workload_table():
    wl = synth.WORKLOADS["vsa_480p"]
    assert (wl.B, wl.Hh, wl.N, wl.D, wl.topk) == (1, 40, 32760, 128, 32)
    assert synth.WORKLOADS["dense_480p_cfg"].B == 2
    assert synth.WORKLOADS["vsa_720p"].N == 75600
    assert synth.WORKLOADS["dense_512_iid"].structured is False
    assert pytest.approx(synth.WORKLOADS["dense_512_iid"].scale) == 0.125


def test_gate_recipe():
    wl = synth.small_workload("g", 2, 3, 5, 6, 7, 128, seed=9)
    g = synth.make_gate(wl)
    assert g.shape == (2, 3, 210, 128) and g.dtype == np.uint16
    x = synth.bits_to_f64(g)
    assert x.min() >= 0.0 and x.max() <= 1.0
    assert abs(x.mean() - 0.5) < 0.01
    assert np.array_equal(synth.make_gate_slice(wl, 1, 2), g[1, 2])
    assert not np.array_equal(g[0, 0], g[0, 1])
