"""wf_attn_dense_noalloc (the dense call with the library's static per-GPU scratch, for callers
that cannot allocate) against wf_attn_dense through the C ABI: the same kernels on the same
inputs, so the outputs must match bit for bit -- on two calls in a row, the second on a smaller
input (the scratch keeps the first call's contents), and after a larger call through the
ordinary entry point.  Sizes beyond the scratch are refused with nothing enqueued."""
import numpy as np
import pytest

import oracle
import synth
from wf_testutil import assert_close, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def _pair(wf, wl):
    import torch
    q, k, v = (to_device(x) for x in synth.make_qkv(wl))
    shape = (wl.B, wl.Hh, wl.N, wl.D)
    want_o = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    want_l = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    wf.wf_attn_dense(q, k, v, out=want_o, lse=want_l)
    got_o = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    got_l = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    wf.wf_attn_dense_noalloc(q, k, v, got_o, got_l)
    torch.cuda.synchronize()
    return (q, k, v), (want_o, want_l), (got_o, got_l)


def test_noalloc_matches_workspace_call_twice(wf):
    import torch
    # first call: 12 heads of the 480p grid (100 MiB of scratch), second: a smaller ragged one
    for wl in (synth.small_workload("noalloc_big", 1, 12, 21, 30, 52, 128, structured=True, seed=301),
               synth.small_workload("noalloc_small", 2, 3, 5, 7, 11, 64, structured=True, seed=302)):
        log(f"dense noalloc B={wl.B} Hh={wl.Hh} N={wl.N} D={wl.D}")
        (q, k, v), (wo, wl_), (go, gl) = _pair(wf, wl)
        assert not torch.isnan(go).any() and not torch.isnan(gl).any()
        assert torch.equal(go, wo) and torch.equal(gl, wl_), "static-scratch call differs from the workspace call"
        ref, _ = oracle.attention(synth.bits_to_f64(synth.make_slice(wl, "q", 0, 0)),
                                  synth.bits_to_f64(synth.make_slice(wl, "k", 0, 0)),
                                  synth.bits_to_f64(synth.make_slice(wl, "v", 0, 0)), wl.scale,
                                  rows=np.arange(min(wl.N, 512)))
        assert_close(go[0, 0, :min(wl.N, 512)].cpu().numpy(), ref, "noalloc O b0 h0 vs oracle")


def test_noalloc_refuses_sizes_beyond_the_scratch(wf):
    import torch
    wl = synth.small_workload("noalloc_limit", 1, 17, 21, 30, 52, 128, structured=False, seed=303)
    q = torch.zeros((wl.B, wl.Hh, wl.N, wl.D), dtype=torch.bfloat16, device="cuda")
    o = torch.full((wl.B, wl.Hh, wl.N, wl.D), 7.0, dtype=torch.float32, device="cuda")
    assert wf.dense_workspace_bytes(wl.B, wl.Hh, wl.N, wl.D) > (128 << 20)
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_dense_noalloc(q, q, q, o)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (o == 7.0).all(), "a refused call must not write"
