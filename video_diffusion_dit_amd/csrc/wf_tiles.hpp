// Tile geometry and copy-offset arithmetic shared by the kernels, in plain C++
// so that the host (and a CPU test built with g++) can evaluate exactly what
// the device computes: LDS swizzles, per-lane global offsets of the
// global -> LDS tile copies, and the bounded byte offset of a key cube inside
// one head's cube-ordered K or V^T region.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define WF_HD __host__ __device__
#else
#define WF_HD
#endif

namespace wf {

// Key order used for V^T tiles inside every group of 16 keys: keys 4..7 and
// 8..11 trade places (bits 2 and 3 of the index swap; an involution).  It is
// the order in which a 32x32 MFMA result holds its rows in one lane pair, so
// the probabilities feed the PV product straight from the score registers.
WF_HD constexpr int perm16(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }

// A K tile is [64 keys][D] bf16 and a V^T tile [D][64 keys] bf16, both
// unpadded.  Each 16-byte chunk is XOR-swizzled within its row so that the 16
// lanes of one ds_read_b128 quarter-wave (one chunk of 16 consecutive rows)
// hit 16 distinct 16-byte bank groups of gfx950's 64-bank LDS.
template <int D>
struct Swz {
  static constexpr int KB = 64 * D * 2;  // K tile bytes
  static constexpr int VB = D * 64 * 2;  // V^T tile bytes
  static constexpr int KCPR = D / 8;     // 16-byte chunks per K row
  WF_HD static constexpr int kslot(int r, int c) { return KCPR == 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7)); }
  WF_HD static constexpr int vslot(int d, int c) { return c ^ ((d >> 1) & 7); }
};

// A V tile stored like a K tile, [64 keys][128] bf16 (no transpose), for P V
// operands read with the gfx950 LDS transpose read ds_read_b64_tr_b16.  That
// instruction works on each group of 16 lanes: lane s of the group supplies
// the address of 4 consecutive bf16 (8 bytes), and lane i of the group
// receives element i % 4 of the chunks of lanes i / 4, 4 + i / 4, 8 + i / 4
// and 12 + i / 4, in that order (measured on gfx950).  The P V MFMA's A
// operand for key step ks (16 keys) and head-dim block b (32 dims) is
// V^T[32 b + j][keys of the probability layout], lane (j, h) element t being
// key 16 ks + 8 (t / 4) + 4 h + t % 4 -- the order in which the score
// registers hold P, so no key permutation is stored.  Two transpose reads
// (r = t / 4) give the 8 elements: lane L = 16 g + 4 e + q (g = group, e, q
// in 0..3) reads row 16 ks + 8 r + 4 (g / 2) + e at dims 32 b + 16 (g % 2) +
// 4 q .. + 3.  The 16-byte chunk c of row r sits at chunk slot
// c ^ (4 (r % 4) + (r / 4) % 4) of the row, which puts the 32 lanes of each
// half wavefront on 64 distinct LDS banks.
struct VtrSwz {
  WF_HD static constexpr int slot(int r, int c) { return c ^ (4 * (r & 3) + ((r >> 2) & 3)); }
  // lane-dependent part of the transpose-read byte offset: row 4 (g / 2) + e, slot bits
  // 4 e + ((2 (g % 2) + q / 2) ^ (g / 2)), half q % 2 of the chunk
  WF_HD static constexpr uint32_t lane_base(int lane) {
    const int g = (lane >> 4) & 3, e = (lane >> 2) & 3, q = lane & 3;
    return (uint32_t)((4 * (g >> 1) + e) * 256 + (4 * e + ((2 * (g & 1) + (q >> 1)) ^ (g >> 1))) * 16 + (q & 1) * 8);
  }
  // byte offset in the tile of transpose read r of key step ks and dim block b
  WF_HD static constexpr uint32_t offset(uint32_t base, int ks, int b, int r) {
    return (base ^ (uint32_t)((4 * b + 2 * r) * 16)) + (uint32_t)((16 * ks + 8 * r) * 256);
  }
};

// Global -> LDS tile copies by NWC wavefronts.  Wavefront w copies K pieces
// g = i * NWC + w (i < KPW), each 1 KiB of the K tile's LDS image: lane L
// fetches the 16-byte chunk that belongs at LDS byte g * 1024 + 16 L under the
// K swizzle.  The swizzle depends on the row only through r & 15, so the
// lane's global offset repeats with period KPER pieces up to a uniform step of
// KSTEP bytes; V^T pieces likewise repeat every piece up to a uniform step of
// NWC * 8 rows.
template <int D, int NWC>
struct CopyGeom {
  static constexpr int CPR = Swz<D>::KCPR, RPP = 64 / CPR;  // 16-byte chunks per K row, K rows per piece
  static constexpr int KPW = Swz<D>::KB / 1024 / NWC, VPW = Swz<D>::VB / 1024 / NWC;
  static constexpr int KPER = (NWC * RPP) % 16 == 0 ? 1 : (2 * NWC * RPP) % 16 == 0 ? 2 : 4;
  static constexpr int KSTEP = KPER * NWC * 1024;  // global bytes between K pieces i and i + KPER
  static_assert(KPW % KPER == 0, "pieces per wavefront");
  static_assert((NWC * 8) % 16 == 0, "V^T swizzle must repeat every piece");
  // per-lane global byte offset of K piece i (i < KPER) of wavefront w, inside one K tile
  WF_HD static constexpr uint32_t k_lane(int i, int w, int lane) {
    return (uint32_t)(((i * NWC + w) * 64 + lane) / CPR * D * 2 +
                      Swz<D>::kslot(((i * NWC + w) * 64 + lane) / CPR, ((i * NWC + w) * 64 + lane) % CPR) * 16);
  }
  // uniform byte step of K piece i past its lane offset k_lane(i % KPER, ...)
  WF_HD static constexpr uint32_t k_step(int i) { return (uint32_t)((i / KPER) * KSTEP); }
  // per-lane global byte offset of V^T piece 0 of wavefront w (row stride vld elements)
  WF_HD static constexpr uint32_t v_lane(int w, int lane, int vld) {
    return (uint32_t)((w * 8 + lane / 8) * vld * 2 + Swz<D>::vslot(w * 8 + lane / 8, lane % 8) * 16);
  }
  // uniform byte step of V^T piece i
  WF_HD static constexpr uint32_t v_step(int i, int vld) { return (uint32_t)(i * NWC * 8 * vld * 2); }
};

// Byte offset of key cube `cube` inside one head's cube-ordered region of C
// cubes of cube_bytes each.  An index outside [0, C) -- a bad caller plan --
// maps to C * cube_bytes, the end of the region: the copies address their
// buffer descriptors at the head with exactly that extent and put this offset
// into the per-lane (range-checked) offset, so such a cube reads zeros
// instead of memory outside the region.
WF_HD constexpr uint32_t cube_offset(int cube, int C, uint32_t cube_bytes) {
  return (uint32_t)cube < (uint32_t)C ? (uint32_t)cube * cube_bytes : (uint32_t)C * cube_bytes;
}

}  // namespace wf
