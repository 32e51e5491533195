"""ctypes binding of libwfattn.so (declarations in include/wf_attn.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory (outputs, workspaces)
and the current HIP stream.  There is no fallback: if the library is not
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# WF_LIB_PATH selects another build of the same library (the host-sanitizer build the CPU tests
# make); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("WF_LIB_PATH") or os.path.join(_HERE, "libwfattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m video_diffusion_dit_amd.build` "
                      "(or __graft_entry__.build()); there is no other implementation to fall back to")

lib = ctypes.CDLL(LIB_PATH)

_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_SIGS = {
    "wf_status_string": (ctypes.c_char_p, [_i32]),
    "wf_last_error_detail": (ctypes.c_char_p, []),
    "wf_abi_version": (_i32, []),
    "wf_attn_dense_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "wf_attn_dense": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "wf_attn_dense_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "wf_attn_dense_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp]),
    "wf_vsa_fine_ex": (_i32, [_vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp, _vp]),
    "wf_vsa_num_cubes": (_i32, [_i32, _i32, _i32]),
    "wf_vsa_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "wf_vsa_coarse_topk": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                  _vp, _vp, _vp, _sz, _vp]),
    "wf_vsa_fine": (_i32, [_vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp]),
    "wf_vsa": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp,
                      _vp, _sz, _vp]),
    "wf_vsa_fine_gated": (_i32, [_vp, _sz, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                 _vp, _vp, _vp, _vp]),
    "wf_rope_qk": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_double, _i32,
                          _vp]),
    "wf_vsa_coarse_topk_rope": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                       ctypes.c_double, _i32, _vp, _vp, _vp, _sz, _vp]),
    "wf_sta_workspace_bytes": (_sz, [_i32] * 9),
    "wf_sta": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp, _vp, _vp,
                      _vp, _sz, _vp]),
    "wf_profile_enable": (_i32, [_i32]),
    "wf_profile_query": (_i32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                ctypes.POINTER(ctypes.c_double)]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype, _fn.argtypes = _res, _args

WF_OK, WF_ERR_INVALID_ARG, WF_ERR_UNSUPPORTED, WF_ERR_WORKSPACE, WF_ERR_BAD_INDEX, WF_ERR_HIP = range(6)
# softmax reference policies (wf_attn.h)
WF_SOFTMAX_GUARDED, WF_SOFTMAX_RUNNING_MAX, WF_SOFTMAX_FIXED_FIRST_TILE = range(3)


class WfError(RuntimeError):
    """A non-zero wf_status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        name = lib.wf_status_string(status).decode()
        detail = lib.wf_last_error_detail().decode()
        super().__init__(f"{where}: {name}: {detail}")


def _check(status: int, where: str) -> None:
    if status != WF_OK:
        raise WfError(status, where)


def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _expect(t, name: str, shape, dtype, device) -> None:
    """The library sees raw pointers only: every tensor handed to it is checked here for device,
    dtype, layout and exact shape, so a wrong tensor raises instead of being read out of bounds."""
    if t is None:
        return
    if (not t.is_cuda or t.device != device or t.dtype != dtype or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         + ("" if t.is_contiguous() else " (not contiguous)"))


def _expect_workspace(ws, device) -> None:
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous() or ws.dim() != 1:
        raise ValueError(f"the workspace must be a contiguous 1-D CUDA tensor on {device}")


def _qkv_check(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 CUDA tensor [B, Hh, N, D]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def num_cubes(T: int, H: int, W: int) -> int:
    return lib.wf_vsa_num_cubes(T, H, W)


def dense_workspace_bytes(B: int, Hh: int, N: int, D: int) -> int:
    return lib.wf_attn_dense_workspace_bytes(B, Hh, N, D)


def vsa_workspace_bytes(B: int, Hh: int, T: int, H: int, W: int, D: int) -> int:
    return lib.wf_vsa_workspace_bytes(B, Hh, T, H, W, D)


def _workspace(nbytes: int, device, given=None):
    torch = _torch()
    if given is not None:
        return given
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def wf_attn_dense(q, k, v, scale: Optional[float] = None, with_lse: bool = False,
                  out=None, lse=None, workspace=None, softmax_mode: int = WF_SOFTMAX_GUARDED):
    """Dense attention through wf_attn_dense (wf_attn_dense_ex for another softmax policy).

    Returns (o fp32 [B,Hh,N,D], lse or None).
    """
    torch = _torch()
    _qkv_check(q, k, v)
    B, Hh, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hh, N, D), dtype=torch.float32, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    _expect(out, "out", (B, Hh, N, D), torch.float32, q.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, q.device)
    ws = _workspace(dense_workspace_bytes(B, Hh, N, D), q.device, workspace)
    _expect_workspace(ws, q.device)
    if softmax_mode == WF_SOFTMAX_GUARDED:
        _check(lib.wf_attn_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                 B, Hh, N, D, scale, ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream_handle(q.device)), "wf_attn_dense")
    else:
        _check(lib.wf_attn_dense_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                    B, Hh, N, D, scale, int(softmax_mode), ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream_handle(q.device)), "wf_attn_dense_ex")
    return out, lse


def wf_attn_dense_noalloc(q, k, v, out, lse=None, scale: Optional[float] = None):
    """Dense attention through wf_attn_dense_noalloc: the library's static per-GPU scratch holds the
    transposed V, so the call allocates nothing.  out (and lse) must be given."""
    torch = _torch()
    _qkv_check(q, k, v)
    B, Hh, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _expect(out, "out", (B, Hh, N, D), torch.float32, q.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, q.device)
    _check(lib.wf_attn_dense_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                     B, Hh, N, D, scale, _stream_handle(q.device)), "wf_attn_dense_noalloc")
    return out, lse


def wf_rope_qk(q, k, grid, theta: float = 10000.0, precision: int = 32, q_out=None, k_out=None):
    """3D RoPE of q and k through wf_rope_qk (precision 32 or 64).  Returns (q_rot, k_rot), bf16.

    Pass q_out=q, k_out=k to rotate in place.
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 CUDA tensor [B, Hh, N, D]")
    if q.shape != k.shape or q.device != k.device:
        raise ValueError(f"q, k differ: {tuple(q.shape)} on {q.device}, {tuple(k.shape)} on {k.device}")
    T, H, W = grid
    B, Hh, N, D = q.shape
    if N != T * H * W:
        raise ValueError(f"N = {N} but the grid has {T * H * W} tokens")
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _expect(q_out, "q_out", q.shape, torch.bfloat16, q.device)
    _expect(k_out, "k_out", k.shape, torch.bfloat16, q.device)
    _check(lib.wf_rope_qk(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), B, Hh, T, H, W, D,
                          float(theta), int(precision), _stream_handle(q.device)), "wf_rope_qk")
    return q_out, k_out


def wf_vsa_coarse_topk(q, k, v, grid, topk: int, scale: Optional[float] = None,
                       with_scores: bool = False, idx=None, scores=None, workspace=None,
                       rope_theta: Optional[float] = None, rope_precision: int = 32):
    """VSA coarse stage through wf_vsa_coarse_topk (wf_vsa_coarse_topk_rope when rope_theta is given).

    grid = (T, H, W).  Returns (idx int32 [B,Hh,C,topk], scores or None,
    workspace) -- pass the workspace on to wf_vsa_fine.
    """
    torch = _torch()
    _qkv_check(q, k, v)
    T, H, W = grid
    B, Hh, N, D = q.shape
    if N != T * H * W:
        raise ValueError(f"N = {N} but the grid has {T * H * W} tokens")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    C = num_cubes(T, H, W)
    if idx is None:
        idx = torch.empty((B, Hh, C, max(topk, 1)), dtype=torch.int32, device=q.device)
    if with_scores and scores is None:
        scores = torch.empty((B, Hh, C, C), dtype=torch.float32, device=q.device)
    _expect(idx, "idx", (B, Hh, C, max(topk, 1)), torch.int32, q.device)  # topk < 1: the library says why
    _expect(scores, "scores", (B, Hh, C, C), torch.float32, q.device)
    ws = _workspace(vsa_workspace_bytes(B, Hh, T, H, W, D), q.device, workspace)
    _expect_workspace(ws, q.device)
    if rope_theta is None:
        _check(lib.wf_vsa_coarse_topk(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hh, T, H, W, D, scale,
                                      topk, idx.data_ptr(), _ptr(scores), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream_handle(q.device)),
               "wf_vsa_coarse_topk")
    else:
        _check(lib.wf_vsa_coarse_topk_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hh, T, H, W, D,
                                           scale, topk, float(rope_theta), int(rope_precision),
                                           idx.data_ptr(), _ptr(scores),
                                           ws.data_ptr(), ws.numel() * ws.element_size(),
                                           _stream_handle(q.device)), "wf_vsa_coarse_topk_rope")
    return idx, scores, ws


def wf_vsa(q, k, v, grid, topk: int, scale: Optional[float] = None, with_lse: bool = False, idx=None,
           out=None, lse=None, workspace=None, gate=None, o_coarse=None):
    """VSA in one call through wf_vsa (coarse stage and fine stage, no cube-ordered copies of Q and K;
    with a gate, the gated coarse branch too).

    grid = (T, H, W).  Returns (o, lse or None, idx int32 [B,Hh,C,topk]).
    """
    torch = _torch()
    _qkv_check(q, k, v)
    T, H, W = grid
    B, Hh, N, D = q.shape
    if N != T * H * W:
        raise ValueError(f"N = {N} but the grid has {T * H * W} tokens")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    C = num_cubes(T, H, W)
    if idx is None:
        idx = torch.empty((B, Hh, C, max(topk, 1)), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, Hh, N, D), dtype=torch.float32, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    _expect(idx, "idx", (B, Hh, C, max(topk, 1)), torch.int32, q.device)  # topk < 1: the library says why
    _expect(out, "out", (B, Hh, N, D), torch.float32, q.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, q.device)
    _expect(gate, "gate", (B, Hh, N, D), torch.bfloat16, q.device)
    _expect(o_coarse, "o_coarse", (B, Hh, C, D), torch.float32, q.device)
    ws = _workspace(vsa_workspace_bytes(B, Hh, T, H, W, D), q.device, workspace)
    _expect_workspace(ws, q.device)
    _check(lib.wf_vsa(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hh, T, H, W, D, scale, topk, idx.data_ptr(),
                      _ptr(gate), out.data_ptr(), _ptr(lse), _ptr(o_coarse), ws.data_ptr(),
                      ws.numel() * ws.element_size(), _stream_handle(q.device)), "wf_vsa")
    return out, lse, idx


def wf_vsa_fine(workspace, idx, shape, grid, scale: Optional[float] = None, with_lse: bool = False,
                out=None, lse=None, softmax_mode: int = WF_SOFTMAX_GUARDED):
    """VSA fine stage through wf_vsa_fine (wf_vsa_fine_ex for another softmax policy).

    shape = (B, Hh, N, D).  Returns (o, lse or None).
    """
    torch = _torch()
    B, Hh, N, D = shape
    T, H, W = grid
    if idx.dim() != 4:
        raise ValueError("idx must be a contiguous int32 tensor [B, Hh, C, topk]")
    if N != T * H * W:
        raise ValueError(f"N = {N} but the grid has {T * H * W} tokens")
    _expect(idx, "idx", (B, Hh, num_cubes(T, H, W), idx.shape[3]), torch.int32, idx.device)
    _expect_workspace(workspace, idx.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hh, N, D), dtype=torch.float32, device=idx.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=idx.device)
    _expect(out, "out", (B, Hh, N, D), torch.float32, idx.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, idx.device)
    if softmax_mode == WF_SOFTMAX_GUARDED:
        _check(lib.wf_vsa_fine(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               idx.data_ptr(), B, Hh, T, H, W, D, scale, idx.shape[3], out.data_ptr(),
                               _ptr(lse), _stream_handle(idx.device)), "wf_vsa_fine")
    else:
        _check(lib.wf_vsa_fine_ex(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  idx.data_ptr(), B, Hh, T, H, W, D, scale, idx.shape[3], int(softmax_mode),
                                  out.data_ptr(), _ptr(lse), _stream_handle(idx.device)), "wf_vsa_fine_ex")
    return out, lse


def wf_vsa_fine_gated(workspace, idx, gate, grid, scale: Optional[float] = None,
                      with_lse: bool = False, with_coarse: bool = False, out=None, lse=None,
                      o_coarse=None):
    """VSA fine stage plus the gated coarse branch through wf_vsa_fine_gated.

    gate: bf16 [B, Hh, N, D] on the device.  Returns (o, lse or None, o_coarse
    [B, Hh, C, D] or None).
    """
    torch = _torch()
    if not gate.is_cuda or gate.dtype != torch.bfloat16 or not gate.is_contiguous() or gate.dim() != 4:
        raise ValueError("gate must be a contiguous 4-D bfloat16 CUDA tensor [B, Hh, N, D]")
    if idx.dim() != 4:
        raise ValueError("idx must be a contiguous int32 tensor [B, Hh, C, topk]")
    B, Hh, N, D = gate.shape
    T, H, W = grid
    if N != T * H * W:
        raise ValueError(f"the gate has N = {N} tokens but the grid has {T * H * W}")
    C = num_cubes(T, H, W)
    _expect(idx, "idx", (B, Hh, C, idx.shape[3]), torch.int32, gate.device)
    _expect_workspace(workspace, gate.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hh, N, D), dtype=torch.float32, device=gate.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=gate.device)
    if with_coarse and o_coarse is None:
        o_coarse = torch.empty((B, Hh, C, D), dtype=torch.float32, device=gate.device)
    _expect(out, "out", (B, Hh, N, D), torch.float32, gate.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, gate.device)
    _expect(o_coarse, "o_coarse", (B, Hh, C, D), torch.float32, gate.device)
    _check(lib.wf_vsa_fine_gated(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 idx.data_ptr(), gate.data_ptr(), B, Hh, T, H, W, D, scale, idx.shape[3],
                                 out.data_ptr(), _ptr(lse), _ptr(o_coarse), _stream_handle(gate.device)),
           "wf_vsa_fine_gated")
    return out, lse, o_coarse


def wf_sta(q, k, v, grid, window, scale: Optional[float] = None, with_lse: bool = False,
           with_plan: bool = False, out=None, lse=None, workspace=None):
    """Sliding-tile attention through wf_sta.  window = (wt, wh, ww) in 6x8x8-token tiles; grid is
    one of the two tuned grids (36, 48, 48) and (18, 48, 80) (the library refuses any other).

    Returns (o, lse or None, plan int32 [tiles, wt*wh*ww] or None).
    """
    torch = _torch()
    _qkv_check(q, k, v)
    T, H, W = grid
    wt, wh, ww = window
    B, Hh, N, D = q.shape
    if N != T * H * W:
        raise ValueError(f"N = {N} but the grid has {T * H * W} tokens")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hh, N, D), dtype=torch.float32, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    tiles = (T // 6) * (H // 8) * (W // 8)
    plan = (torch.empty((max(tiles, 1), wt * wh * ww), dtype=torch.int32, device=q.device)
            if with_plan else None)
    _expect(out, "out", (B, Hh, N, D), torch.float32, q.device)
    _expect(lse, "lse", (B, Hh, N), torch.float32, q.device)
    ws = _workspace(lib.wf_sta_workspace_bytes(B, Hh, T, H, W, D, wt, wh, ww), q.device, workspace)
    _expect_workspace(ws, q.device)
    _check(lib.wf_sta(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hh, T, H, W, D, scale, wt, wh, ww,
                      out.data_ptr(), _ptr(lse), _ptr(plan), ws.data_ptr(), ws.numel() * ws.element_size(),
                      _stream_handle(q.device)), "wf_sta")
    return out, lse, plan


def vsa(q, k, v, grid, topk: int, scale: Optional[float] = None, with_lse: bool = False,
        with_scores: bool = False):
    """Both VSA stages.  Returns dict(idx, o, lse, scores)."""
    idx, scores, ws = wf_vsa_coarse_topk(q, k, v, grid, topk, scale, with_scores)
    o, lse = wf_vsa_fine(ws, idx, tuple(q.shape), grid, scale, with_lse)
    return dict(idx=idx, o=o, lse=lse, scores=scores)


def profile_enable(on: bool) -> None:
    _check(lib.wf_profile_enable(1 if on else 0), "wf_profile_enable")


def profile_query(name: str):
    """(launches, total_ms) of the kernel `name` since profile_enable(True)."""
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(lib.wf_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)), "wf_profile_query")
    return n.value, ms.value
