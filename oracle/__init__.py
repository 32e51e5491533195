"""fp64 CPU oracle for video-DiT self-attention, dense and Video Sparse Attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or call anything here.  The HIP
path never does, and this package imports nothing from it: the two share no
code, headers, tables or helpers (the seeded input generator in ``synth`` is
the only common module, and it holds none of the method's arithmetic).

Sources (cited by page title and section; no code is printed on the pages):

* "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com, Persian), the review of
  Baseten's Wan2.2 work.  Sections used: "Why video attention becomes the
  bottleneck" (dense self-attention over the 30x52x21 token grid, every
  query against every key), "VSA selects cubes" (padding, 4x4x4 cubes,
  coarse stage on cube-mean Q/K, top-k key cubes, fine stage), "Roofline
  analysis set the 3.35 ms target" (tile count, FLOP and byte conventions),
  "Fixed-max softmax is a numerical contract" (running-max online softmax
  is exact and stable; a fixed constant can overflow).
* "Wan2.1 acceleration" blog (bafh001.com), section 4.2: attention is
  called non-causally, with QK^T, softmax and PV fused block-wise on chip.
* "推理优化" (Inference optimization, WorldFoundry docs), section "Exact or
  numerically equivalent Wan kernels", entry fused_rope: a fused 3D RoPE
  with an fp32 or fp64 rotation (oracle/rope.py states the definition
  adopted, since the page gives no frequencies); and, in its approximate
  attention section, entry "sta", weight-free sliding-tile attention accepted
  only on two tuned grids (oracle/sta.py states the 6x8x8 tile and the window
  definition adopted).

Readings taken where the pages are silent are listed in each function's
docstring.  All functions take float64 numpy arrays (bf16 inputs widened
exactly) and return float64.

Pins: every function here is checked in ``tests/test_oracle.py`` against
brute-force loops, closed forms, library routines (scipy's logsumexp) and
the numbers the pages print; see that file's header for the map.
"""
from .dense import attention, attention_heads
from .rope import axis_split, grid_positions, angles, rotate, round_bf16, rope, rope_bf16
from .sta import TILE, TUNED_GRIDS, tile_grid, tile_tokens, window_start, sta_plan, sta
from .vsa import (CUBE, geometry, cube_layout, pool, coarse_scores, select_topk,
                  near_tie_tolerance, fine, vsa, coarse_output, gated, flops_fine, kv_stream_bytes)

__all__ = ["attention", "attention_heads", "CUBE", "geometry", "cube_layout", "pool",
           "coarse_scores", "select_topk", "near_tie_tolerance", "fine", "vsa",
           "coarse_output", "gated", "flops_fine", "kv_stream_bytes", "axis_split", "grid_positions",
           "angles", "rotate", "round_bf16", "rope", "rope_bf16", "TILE", "TUNED_GRIDS", "tile_grid",
           "tile_tokens", "window_start", "sta_plan", "sta"]
