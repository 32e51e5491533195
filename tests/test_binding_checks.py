"""The Python binding refuses tensors that do not match what it passes to the library (the C ABI
sees raw pointers only), so a wrong shape, dtype or device raises instead of being read or written
out of bounds.  Needs the GPU for device tensors; no kernel runs for the refused calls."""
import pytest

import synth
from wf_testutil import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wf():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_dit_amd as wf
    return wf


def test_binding_refuses_mismatched_tensors(wf):
    import torch
    wl = synth.small_workload("binding", 1, 2, 5, 6, 7, 128, structured=True, seed=130, topk=3)
    log("binding checks 5x6x7")
    q, k, v = (to_device(x) for x in synth.make_qkv(wl))
    grid, C = (5, 6, 7), wf.num_cubes(5, 6, 7)
    with pytest.raises(ValueError):   # dense: output of the wrong shape
        wf.wf_attn_dense(q, k, v, out=torch.empty((1, 2, 209, 128), device="cuda"))
    with pytest.raises(ValueError):   # dense: lse of the wrong dtype
        wf.wf_attn_dense(q, k, v, lse=torch.empty((1, 2, 210), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):   # coarse: idx with too few cubes
        wf.wf_vsa_coarse_topk(q, k, v, grid, 3, idx=torch.empty((1, 2, C - 1, 3), dtype=torch.int32, device="cuda"))
    idx, _, ws = wf.wf_vsa_coarse_topk(q, k, v, grid, 3)
    with pytest.raises(ValueError):   # fine: token count differs from the grid
        wf.wf_vsa_fine(ws, idx, (1, 2, 209, 128), grid)
    with pytest.raises(ValueError):   # fine: idx on the host
        wf.wf_vsa_fine(ws, idx.cpu(), (1, 2, 210, 128), grid)
    with pytest.raises(ValueError):   # gated: gate with another token count
        wf.wf_vsa_fine_gated(ws, idx, q[:, :, :200].contiguous(), grid)
    with pytest.raises(ValueError):   # gated: o_coarse of the wrong shape
        wf.wf_vsa_fine_gated(ws, idx, q, grid, o_coarse=torch.empty((1, 2, C, 64), device="cuda"))
    with pytest.raises(ValueError):   # rope: output of another dtype
        wf.wf_rope_qk(q, k, grid, q_out=torch.empty((1, 2, 210, 128), device="cuda"))
    with pytest.raises(ValueError):   # sta: lse of the wrong shape
        wf.wf_sta(q, k, v, grid, (1, 1, 1), lse=torch.empty((1, 2), device="cuda"))
    with pytest.raises(ValueError):   # a workspace on the host
        wf.wf_vsa_fine(ws.cpu(), idx, (1, 2, 210, 128), grid)
    o, _ = wf.wf_vsa_fine(ws, idx, (1, 2, 210, 128), grid)   # and the right tensors still work
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
