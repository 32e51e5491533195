// Block arithmetic of the VSA path: block coordinates by multiply-high division, first tokens of
// blocks, and the offsets of the copies that read one 4x4x4 key cube of K and V straight from the
// token grid (the one-call path, which skips the cube-ordered copies of K and V).  Plain C++ for
// host and device, so the arithmetic can be checked on the host.
#pragma once

#include <stdint.h>

#include "wf_tiles.hpp"

namespace wf {

// Division of a block index n < 2^12 by a runtime divisor 1 <= d < 2^20 with one multiply-high:
// with m = ceil(2^32 / d), n * m / 2^32 exceeds n / d by less than n / 2^32 < 1 / d, so its floor
// is floor(n / d).  m = 0 stands for d = 1 (whose m needs 33 bits).
WF_HD constexpr uint32_t div_magic(uint32_t d) {
  return d <= 1 ? 0u : (uint32_t)(((1ull << 32) + d - 1) / d);
}
WF_HD constexpr uint32_t div_by_magic(uint32_t n, uint32_t m) {
  return m ? (uint32_t)(((uint64_t)n * m) >> 32) : n;
}

// First token of the BT x BH x BW block at block coordinates (bt, bh, bw) of a T x H x W token
// grid; cube_first_token_at for 4x4x4 cubes.
template <int BT, int BH, int BW>
WF_HD constexpr uint32_t block_first_token(int bt, int bh, int bw, int H, int W) {
  return (uint32_t)((BT * bt * H + BH * bh) * W + BW * bw);
}
WF_HD constexpr uint32_t cube_first_token_at(int ct, int ch, int cw, int H, int W) {
  return block_first_token<4, 4, 4>(ct, ch, cw, H, W);
}

// Whether slots 32..63 of a BT x BH x BW block of 64 slots (slot s at (s / (BH BW), s / BW % BH,
// s % BW)) are all padding, for a block that extends lt and lh tokens inside the grid along t and
// h (BT or more, BH or more: whole): they are the block's second half along t (BT > 1) or, for
// blocks one token deep, along h.  Every block holds at least one token on each axis.
template <int BT, int BH, int BW>
WF_HD constexpr bool second_half_padded(int lt, int lh) {
  static_assert(BT * BH * BW == 64 && (BT > 1 ? BT % 2 : BH % 2) == 0, "64-slot blocks split along t, or along h");
  return BT > 1 ? lt <= BT / 2 : lh <= BH / 2;
}

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

// The same offsets split into a part shared by the wavefront and a per-lane part, so a copy
// costs one add per piece: piece i of wavefront w starts at token row part grid_row_part and lane
// `lane` adds grid_lane_part, which depends on i only through i % 2 (V selects the V tile's
// swizzle, VtrSwz).  grid_row_part(...) + grid_lane_part<false>(i % 2, ...) equals
// grid_k_offset, and with <true> grid_v_offset_full.
WF_HD constexpr uint32_t grid_row_part(uint32_t first_token, int i, int w, int H, int W) {
  const int sr = 2 * i + w;
  return (first_token + (uint32_t)((sr / 4) * H * W + (sr % 4) * W)) * 256u;
}
template <bool V>
WF_HD constexpr uint32_t grid_lane_part(int i_odd, int w, int lane) {
  const int dw = lane / 16, row = 4 * (2 * i_odd + w) + dw;  // the slot row modulo 16
  return (uint32_t)dw * 256u + (uint32_t)(V ? VtrSwz::slot(row, lane % 16) : Swz<128>::kslot(row, lane % 16)) * 16u;
}

// grid_k_offset for a V tile read by transpose reads: the same pieces and slots, the chunk placed
// under the V tile's swizzle (VtrSwz) -- for a cube inside the grid on every axis.
WF_HD constexpr uint32_t grid_v_offset_full(uint32_t first_token, int i, int w, int lane, int H, int W) {
  const int sr = 2 * i + w, dw = lane / 16;
  const uint32_t tok = first_token + (uint32_t)((sr / 4) * H * W + (sr % 4) * W + dw);
  return tok * 256u + (uint32_t)VtrSwz::slot(4 * sr + dw, lane % 16) * 16u;
}
// The same for any cube: a slot outside the grid (the cube extends lt, lh, lw slots inside it
// along t, h, w) gets head_bytes, which the range check turns into zeros, as the cube-ordered copy
// holds there -- its probability is zero, and a zero row keeps it so whatever V holds elsewhere.
WF_HD constexpr uint32_t grid_v_offset(uint32_t first_token, int i, int w, int lane, int H, int W, int lt, int lh,
                                       int lw, uint32_t head_bytes) {
  const int sr = 2 * i + w, dw = lane / 16;
  return (sr / 4 < lt && sr % 4 < lh && dw < lw) ? grid_v_offset_full(first_token, i, w, lane, H, W) : head_bytes;
}

}  // namespace wf
