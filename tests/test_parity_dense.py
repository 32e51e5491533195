"""Dense attention on the GPU (through the C ABI) against the fp64 oracle.

Small shapes are compared on every output; a D = 64 case over several query
tiles and a 1M-token head on sampled rows.  Outputs are poisoned (NaN) before
every call.  The production shapes (12 heads and the CFG pair x 40 heads at
480p, the CFG pair at 720p) are checked whole in test_parity_full.py.
"""
import math

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


def run_dense(wf, q, k, v, scale=None):
    """One call on outputs poisoned first (NaN): every row must be written."""
    import torch
    B, Hh, N, D = q.shape
    o = torch.full((B, Hh, N, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hh, N), float("nan"), dtype=torch.float32, device="cuda")
    wf.wf_attn_dense(to_device(q), to_device(k), to_device(v), scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "output rows never written"
    return o, lse


def oracle_heads(wl, q, k, v, heads, rows=None):
    def one(bh):
        b, h = bh
        return oracle.attention(synth.bits_to_f64(q[b, h]), synth.bits_to_f64(k[b, h]),
                                synth.bits_to_f64(v[b, h]), wl.scale, rows)
    return dict(zip(heads, pmap(one, heads)))


def sample_rows(N, rng, n_random=192):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 65, N - 64,
             N - 33, N - 32, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(rng.choice(N, size=min(n_random, N), replace=False).tolist())
    return np.array(sorted(rows))


def test_dense_512_iid_all_outputs(wf):
    wl = synth.WORKLOADS["dense_512_iid"]
    log(f"dense {wl.name} B={wl.B} Hh={wl.Hh} N={wl.N} D={wl.D}")
    q, k, v = synth.make_qkv(wl)
    o, lse = run_dense(wf, q, k, v)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.Hh)]
    ref = oracle_heads(wl, q, k, v, heads)
    for b, h in heads:
        assert_close(o[b, h], ref[(b, h)][0], f"O b{b} h{h}")
        assert errors(lse[b, h], ref[(b, h)][1])[0] <= LSE_MAX_ABS


@pytest.mark.parametrize("N,D,B,Hh", [(1, 128, 1, 1), (37, 64, 2, 3), (64, 128, 1, 2), (65, 128, 1, 2),
                                      (200, 64, 1, 1), (333, 128, 2, 2), (1000, 128, 1, 3)])
def test_dense_ragged_small(wf, N, D, B, Hh):
    wl = synth.small_workload("ragged", B, Hh, 1, 1, N, D, structured=True, seed=N + D)
    log(f"dense ragged B={B} Hh={Hh} N={N} D={D}")
    q, k, v = synth.make_qkv(wl)
    o, lse = run_dense(wf, q, k, v)
    heads = [(b, h) for b in range(B) for h in range(Hh)]
    ref = oracle_heads(wl, q, k, v, heads)
    for b, h in heads:
        assert_close(o[b, h], ref[(b, h)][0], f"O b{b} h{h}")
        assert errors(lse[b, h], ref[(b, h)][1])[0] <= LSE_MAX_ABS


def test_dense_closed_forms_on_gpu(wf):
    """V = 1 gives O = 1; Q = 0 gives the mean of V (exact closed forms, no oracle)."""
    wl = synth.small_workload("cf", 1, 2, 3, 10, 31, 128, structured=True, seed=5)
    log("dense closed forms N=930 D=128")
    q, k, v = synth.make_qkv(wl)
    ones = np.full_like(v, 0x3F80)  # bf16 1.0
    o, _ = run_dense(wf, q, k, ones)
    assert np.abs(o - 1.0).max() <= 1e-5
    zeros = np.zeros_like(q)
    o, lse = run_dense(wf, zeros, k, v)
    mean_v = synth.bits_to_f64(v).mean(axis=2, keepdims=True)
    assert_close(o, np.broadcast_to(mean_v, o.shape), "Q=0 mean(V)", max_abs=2e-3, mean_abs=5e-4)
    assert np.abs(lse - math.log(wl.N)).max() <= 1e-4


def test_dense_large_values_stay_finite(wf):
    """|V| near 1e30 and logits near 1e3 together: the accumulators must not overflow."""
    wl = synth.small_workload("bigv", 1, 1, 4, 8, 16, 128, structured=True, seed=10)
    log("dense large V N=512 D=128")
    q, k, v = synth.make_qkv(wl)
    qb = synth.bf16_bits(synth.bits_to_f32(q) * 64.0)
    vb = synth.bf16_bits(synth.bits_to_f32(v) * 1e30)
    o, lse = run_dense(wf, qb, k, vb)
    ref_o, _ = oracle.attention(synth.bits_to_f64(qb[0, 0]), synth.bits_to_f64(k[0, 0]),
                                synth.bits_to_f64(vb[0, 0]), wl.scale)
    assert np.isfinite(o).all()
    assert_close(o[0, 0] / 1e30, ref_o / 1e30, "O large V (scaled by 1e-30)")


def test_dense_large_logits_stay_finite(wf):
    """Q scaled x64 drives logits to ~1e3: a softmax without the running max overflows."""
    wl = synth.small_workload("big", 1, 1, 4, 8, 16, 128, structured=True, seed=9)
    log("dense adversarial logits N=512 D=128")
    q, k, v = synth.make_qkv(wl)
    qf = synth.bits_to_f32(q) * 64.0
    qb = synth.bf16_bits(qf)
    o, lse = run_dense(wf, qb, k, v)
    ref_o, ref_l = oracle.attention(synth.bits_to_f64(qb[0, 0]), synth.bits_to_f64(k[0, 0]),
                                    synth.bits_to_f64(v[0, 0]), wl.scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert ref_l.max() > 500
    assert_close(o[0, 0], ref_o, "O adversarial")


def test_dense_d64_multi_tile_sampled(wf):
    """Head dimension 64 over several query tiles of 256 rows and a ragged key tail
    (grid 9 x 23 x 31 = 6,417 tokens), 2 x 6 heads: every head sampled."""
    wl = synth.small_workload("d64", 2, 6, 9, 23, 31, 64, structured=True, seed=64)
    log(f"dense d64 B={wl.B} Hh={wl.Hh} N={wl.N} D={wl.D} (sampled rows of every head)")
    q, k, v = synth.make_qkv(wl)
    o, lse = run_dense(wf, q, k, v)
    rows = sample_rows(wl.N, np.random.default_rng(wl.seed), n_random=64)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.Hh)]
    ref = oracle_heads(wl, q, k, v, heads, rows)
    for bh in heads:
        assert_close(o[bh][rows], ref[bh][0], f"O b{bh[0]} h{bh[1]} ({rows.size} rows)")
        assert errors(lse[bh][rows], ref[bh][1])[0] <= LSE_MAX_ABS
    assert np.isfinite(o).all()


def test_dense_long_ragged_sampled(wf):
    """One head of 1,044,735 tokens (grid 17 x 241 x 255, ragged last tile): 32-bit
    offsets and buffer extents far beyond the benchmark shapes, sampled rows."""
    wl = synth.small_workload("long", 1, 1, 17, 241, 255, 128, structured=True, seed=41)
    log(f"dense long N={wl.N} D={wl.D} (sampled rows)")
    q, k, v = synth.make_qkv(wl)
    o, lse = run_dense(wf, q, k, v)
    rows = sample_rows(wl.N, np.random.default_rng(wl.seed), n_random=24)
    ref_o, ref_l = oracle.attention(synth.bits_to_f64(q[0, 0]), synth.bits_to_f64(k[0, 0]),
                                    synth.bits_to_f64(v[0, 0]), wl.scale, rows)
    assert_close(o[0, 0][rows], ref_o, f"O ({rows.size} rows)")
    assert errors(lse[0, 0][rows], ref_l)[0] <= LSE_MAX_ABS
    assert np.isfinite(o).all()


def test_dense_concurrent_streams(wf):
    """Calls are reentrant: two streams, each with its own workspace, running at once give the
    same bits as the calls made one after the other."""
    import torch
    wl = synth.small_workload("dense_streams", 1, 6, 9, 11, 13, 128, structured=True, seed=120)
    log("dense on two concurrent streams, 6 heads x 1287 tokens")
    q, k, v = synth.make_qkv(wl)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ref, _ = wf.wf_attn_dense(qd, kd, vd)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for st in (s1, s2):
        with torch.cuda.stream(st):
            outs.append(wf.wf_attn_dense(qd, kd, vd)[0])
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
