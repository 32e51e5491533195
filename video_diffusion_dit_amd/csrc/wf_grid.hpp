// Offsets of the key-tile copies that read one 4x4x4 key cube of K and V straight from the token
// grid (the one-call VSA path, which skips the cube-ordered copies of K and V).  Plain C++ for host and
// device, so the arithmetic can be checked on the host.
#pragma once

#include <stdint.h>

#include "wf_tiles.hpp"

namespace wf {

// First token of cube `cube` of the padded (nt, nh, nw) cube grid of a T x H x W token grid
// (tokens in row-major (t, h, w) order); for an index outside [0, C), N, the head's end.
WF_HD constexpr uint32_t cube_first_token(int cube, int C, int nh, int nw, int H, int W, uint32_t N) {
  return (uint32_t)cube < (uint32_t)C
             ? (uint32_t)((4 * (cube / (nw * nh)) * H + 4 * ((cube / nw) % nh)) * W + 4 * (cube % nw))
             : N;
}

// Byte offset (inside one head's K, D = 128 bf16 per token) that lane `lane` of wavefront w
// (of 2) reads for piece i (of 8) of a key tile: the piece holds cube slots 4 (2i + w) .. +3,
// slot row dt = (2i + w) / 4, dh = (2i + w) % 4, dw = lane / 16, and lane % 16 is the chunk's
// place in the swizzled LDS row (Swz<128>), so the lane fetches chunk kslot(row, lane % 16)
// of its token, exactly what the cube-ordered copy fetches from that slot's row.
WF_HD constexpr uint32_t grid_k_offset(uint32_t first_token, int i, int w, int lane, int H, int W) {
  const int sr = 2 * i + w, dw = lane / 16;
  const uint32_t tok = first_token + (uint32_t)((sr / 4) * H * W + (sr % 4) * W + dw);
  return tok * 256u + (uint32_t)Swz<128>::kslot(4 * sr + dw, lane % 16) * 16u;
}

// The same for a V tile read by transpose reads (VtrSwz): the same pieces and slots, the
// chunk placed under the V tile's swizzle.  A slot outside the grid (the cube's first lt, lh, lw
// slot coordinates along t, h, w are inside it) gets head_bytes, which the range check turns
// into zeros, as the cube-ordered copy holds there: its probability is zero, and a zero row
// keeps it so whatever the other rows of V hold.
WF_HD constexpr uint32_t grid_v_offset(uint32_t first_token, int i, int w, int lane, int H, int W, int lt, int lh,
                                       int lw, uint32_t head_bytes) {
  const int sr = 2 * i + w, dw = lane / 16;
  const uint32_t tok = first_token + (uint32_t)((sr / 4) * H * W + (sr % 4) * W + dw);
  return (sr / 4 < lt && sr % 4 < lh && dw < lw) ? tok * 256u + (uint32_t)VtrSwz::slot(4 * sr + dw, lane % 16) * 16u
                                                   : head_bytes;
}

}  // namespace wf
