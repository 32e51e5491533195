"""3D RoPE on the GPU (through the C ABI) against the fp64 oracle.

In both of the page's precisions (fp64, and fp32 with every product and sum
rounded to fp32) the GPU and the oracle take the same bf16 rounding decision
on the same value, so the rotated Q and K must match the oracle's bit for
bit (ragged grids, W above one 64-token block, more than one group of 8
heads, D = 64 and 128, in place, another frequency base, all 40 heads at
480p).  The RoPE fused into
VSA's gather must give exactly what wf_rope_qk followed by the plain coarse
stage gives, and VSA and dense attention on rotated inputs must match the
oracle run on the oracle's own rotated inputs.
"""
import numpy as np
import pytest

import oracle
import synth
from test_parity_vsa import check_fine, check_scores_and_idx, coarse_ref
from wf_testutil import assert_close, log, pmap, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def bits_of(t):
    """bf16 CUDA tensor -> uint16 bit patterns (numpy)."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


PREC = {32: "fp32", 64: "fp64"}


def oracle_rope_bits(x_bits, T, H, W, theta, prec=32):
    """Oracle rotation of every (b, h) slice of bf16 bits [B, Hh, N, D], as bf16 bits."""
    B, Hh = x_bits.shape[:2]
    out = np.empty_like(x_bits)

    def one(bh):
        b, h = divmod(bh, Hh)
        r = oracle.rope_bf16(synth.bits_to_f64(x_bits[b, h]), T, H, W, theta, PREC[prec])
        out[b, h] = synth.bf16_bits(r.astype(np.float32))   # r is bf16-valued: exact
    pmap(one, range(B * Hh))
    return out


@pytest.mark.parametrize("prec", [32, 64])
@pytest.mark.parametrize("B,Hh,grid,D,theta", [(1, 2, (5, 6, 7), 128, 10000.0), (2, 9, (3, 5, 70), 128, 10000.0),
                                               (1, 3, (4, 4, 4), 64, 10000.0), (1, 1, (1, 1, 1), 128, 10000.0),
                                               (1, 2, (7, 3, 11), 128, 500.0), (2, 3, (2, 9, 130), 64, 10000.0)])
def test_rope_qk_bit_exact(wf, B, Hh, grid, D, theta, prec):
    T, H, W = grid
    wl = synth.small_workload("rope", B, Hh, T, H, W, D, structured=True, seed=70 + T + D)
    log(f"rope B={B} Hh={Hh} grid={grid} D={D} theta={theta} fp{prec}")
    q, k, _ = synth.make_qkv(wl)
    qr, kr = wf.wf_rope_qk(to_device(q), to_device(k), grid, theta, prec)
    for name, got, x in (("q", bits_of(qr), q), ("k", bits_of(kr), k)):
        ref = oracle_rope_bits(x, T, H, W, theta, prec)
        bad = np.count_nonzero(got != ref)
        assert bad == 0, f"{name}: {bad} of {ref.size} bf16 values differ from the oracle"


def test_rope_qk_in_place(wf):
    wl = synth.small_workload("rope_ip", 1, 4, 6, 7, 9, 128, structured=True, seed=77)
    log("rope in place 6x7x9")
    q, k, _ = synth.make_qkv(wl)
    qd, kd = to_device(q), to_device(k)
    qr, kr = wf.wf_rope_qk(qd, kd, (6, 7, 9))
    wf.wf_rope_qk(qd, kd, (6, 7, 9), q_out=qd, k_out=kd)
    assert np.array_equal(bits_of(qd), bits_of(qr)) and np.array_equal(bits_of(kd), bits_of(kr))
    assert np.array_equal(bits_of(qd), oracle_rope_bits(q, 6, 7, 9, 10000.0))


@pytest.mark.parametrize("prec", [32, 64])
def test_rope_qk_480p_all_heads(wf, prec):
    wl = synth.WORKLOADS["vsa_480p"]
    log(f"rope {wl.name} all {wl.Hh} heads fp{prec}")
    q, k, _ = synth.make_qkv(wl)
    qr, kr = wf.wf_rope_qk(to_device(q), to_device(k), (wl.T, wl.H, wl.W), precision=prec)
    for name, got, x in (("q", bits_of(qr), q), ("k", bits_of(kr), k)):
        ref = oracle_rope_bits(x, wl.T, wl.H, wl.W, 10000.0, prec)
        assert np.count_nonzero(got != ref) == 0, name


def fused_vs_separate(wf, wl, q, k, v, prec=32):
    """VSA with the gather's RoPE and VSA after wf_rope_qk: every output must be equal."""
    import torch
    grid, shape = (wl.T, wl.H, wl.W), tuple(q.shape)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    idx_f, s_f, ws_f = wf.wf_vsa_coarse_topk(qd, kd, vd, grid, wl.topk, with_scores=True, rope_theta=10000.0,
                                             rope_precision=prec)
    o_f, l_f = wf.wf_vsa_fine(ws_f, idx_f, shape, grid, with_lse=True)
    qr, kr = wf.wf_rope_qk(qd, kd, grid, precision=prec)
    idx_s, s_s, ws_s = wf.wf_vsa_coarse_topk(qr, kr, vd, grid, wl.topk, with_scores=True)
    o_s, l_s = wf.wf_vsa_fine(ws_s, idx_s, shape, grid, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s) and torch.equal(s_f, s_s)
    assert torch.equal(o_f, o_s) and torch.equal(l_f, l_s)
    return dict(idx=idx_f.cpu().numpy(), scores=s_f.cpu().numpy(), o=o_f.cpu().numpy(), lse=l_f.cpu().numpy())


@pytest.mark.parametrize("grid,topk,Hh,prec", [((5, 6, 7), 3, 2, 32), ((9, 10, 11), 5, 1, 32),
                                                ((13, 6, 21), 9, 2, 32), ((9, 10, 11), 5, 2, 64)])
def test_vsa_rope_small_grids(wf, grid, topk, Hh, prec):
    T, H, W = grid
    wl = synth.small_workload("vsa_rope", 1, Hh, T, H, W, 128, structured=True, seed=80 + T, topk=topk)
    log(f"vsa rope grid={grid} topk={topk} Hh={Hh} fp{prec}")
    q, k, v = synth.make_qkv(wl)
    g = fused_vs_separate(wf, wl, q, k, v, prec)
    qo, ko = oracle_rope_bits(q, T, H, W, 10000.0, prec), oracle_rope_bits(k, T, H, W, 10000.0, prec)
    heads = [(0, h) for h in range(Hh)]
    ref, tok = coarse_ref(wl, qo, ko, heads, topk)
    check_scores_and_idx(g, ref, heads)
    check_fine(wl, qo, ko, v, g, tok, heads)


def test_vsa_rope_480p(wf):
    wl = synth.WORKLOADS["vsa_480p"]
    log(f"vsa rope {wl.name} topk={wl.topk}")
    q, k, v = synth.make_qkv(wl)
    g = fused_vs_separate(wf, wl, q, k, v)
    qo = oracle_rope_bits(q, wl.T, wl.H, wl.W, 10000.0)
    ko = oracle_rope_bits(k, wl.T, wl.H, wl.W, 10000.0)
    heads = [(0, h) for h in range(0, wl.Hh, 3)]
    ref, tok = coarse_ref(wl, qo, ko, heads, wl.topk)
    check_scores_and_idx(g, ref, heads)
    cubes = sorted(np.random.default_rng(81).choice(tok.shape[0], 16, replace=False).tolist() + [0, 623])
    check_fine(wl, qo, ko, v, g, tok, [(0, 6), (0, 33)], cubes)


def test_dense_after_rope(wf):
    wl = synth.small_workload("dense_rope", 1, 2, 6, 7, 9, 128, structured=True, seed=83)
    log("dense after rope 6x7x9")
    q, k, v = synth.make_qkv(wl)
    qr, kr = wf.wf_rope_qk(to_device(q), to_device(k), (wl.T, wl.H, wl.W))
    o, _ = wf.wf_attn_dense(qr, kr, to_device(v))
    o = o.cpu().numpy()
    qo, ko = oracle_rope_bits(q, wl.T, wl.H, wl.W, 10000.0), oracle_rope_bits(k, wl.T, wl.H, wl.W, 10000.0)
    for h in range(2):
        ref, _ = oracle.attention(synth.bits_to_f64(qo[0, h]), synth.bits_to_f64(ko[0, h]),
                                  synth.bits_to_f64(v[0, h]), wl.scale)
        assert_close(o[0, h], ref, f"dense after RoPE h{h}")


def test_rope_error_paths(wf):
    wl = synth.small_workload("rope_err", 1, 1, 2, 3, 4, 128, seed=84)
    q, k, _ = synth.make_qkv(wl)
    qd, kd = to_device(q), to_device(k)
    with pytest.raises(wf.WfError) as e:
        wf.wf_rope_qk(qd, kd, (2, 3, 4), theta=0.0)
    assert e.value.status == 1
    with pytest.raises(wf.WfError) as e:
        wf.wf_rope_qk(qd[..., :96].contiguous(), kd[..., :96].contiguous(), (2, 3, 4))
    assert e.value.status == 2
    with pytest.raises(ValueError):
        wf.wf_rope_qk(qd, kd, (2, 3, 5))
    with pytest.raises(wf.WfError) as e:
        wf.wf_vsa_coarse_topk(qd, kd, qd, (2, 3, 4), 1, rope_theta=float("nan"))
    assert e.value.status == 1
