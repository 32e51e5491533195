"""MI355X-native self-attention over a video DiT's 3D latent token grid.

Dense flash-style attention and Video Sparse Attention (cube gather, coarse
cube scores, per-cube top-k, fine block-sparse attention, gated merge with the
coarse branch), sliding-tile attention over 6x8x8 tiles, with an optional 3D
RoPE of Q and K, as hand-written gfx950 HIP kernels behind the C ABI of
libwfattn.so (include/wf_attn.h).
Importing this package loads the library and fails if it is not built.
"""
from ._binding import (LIB_PATH, WfError, lib, wf_attn_dense, wf_attn_dense_noalloc, wf_vsa, wf_vsa_coarse_topk, wf_vsa_fine,
                       wf_vsa_fine_gated, wf_rope_qk, wf_sta, vsa, num_cubes, dense_workspace_bytes, vsa_workspace_bytes,
                       profile_enable, profile_query)

__all__ = ["LIB_PATH", "WfError", "lib", "wf_attn_dense", "wf_attn_dense_noalloc", "wf_vsa", "wf_vsa_coarse_topk", "wf_vsa_fine",
           "wf_vsa_fine_gated", "wf_rope_qk", "wf_sta", "vsa",
           "num_cubes", "dense_workspace_bytes", "vsa_workspace_bytes", "profile_enable",
           "profile_query"]
