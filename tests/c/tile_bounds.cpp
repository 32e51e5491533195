// Host check of the copy arithmetic the kernels use (wf_tiles.hpp, built here with g++):
//  * every K / V^T tile copy covers each 16-byte chunk of the tile exactly once;
//  * in the fine stage a key cube inside [0, C) is read only from its own 16 KiB, and an
//    index outside [0, C) -- any int, including ones whose byte offset would wrap 32 bits --
//    gets a per-lane offset at or past the end of the head's region, which the buffer
//    descriptor's range check turns into zeros;
//  * the one-call path's K copy from the token grid (wf_grid.hpp) reads, for every real slot of
//    every cube of ragged and even grids, exactly the bytes the cube-ordered copy reads for it,
//    and for a cube index outside [0, C) starts at the head's end; its V copy reads the same
//    token rows, chunks placed under the V tile's swizzle (VtrSwz);
//  * block coordinates by multiply-high division (div_magic) match plain division;
//  * second_half_padded, which lets the fine stage skip work on edge blocks, holds exactly when
//    slots 32..63 are all padding;
//  * the transpose reads of that V tile (VtrSwz offsets, under the lane mapping of gfx950's
//    ds_read_b64_tr_b16) deliver to every lane of every P V MFMA exactly the V^T elements its A
//    operand needs, in the probability registers' key order, and each half wavefront of every
//    read touches 64 distinct LDS banks.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <climits>
#include <vector>

#include "wf_grid.hpp"
#include "wf_tiles.hpp"

static int fails = 0;
#define EXPECT(c, ...)                      \
  do {                                      \
    if (!(c)) {                             \
      if (fails < 10) printf(__VA_ARGS__);  \
      ++fails;                              \
    }                                       \
  } while (0)

template <int D, int NWC>
static void coverage() {
  using G = wf::CopyGeom<D, NWC>;
  const int tile = 64 * D * 2;
  std::vector<int> k(tile / 16, 0), v(tile / 16, 0);
  for (int w = 0; w < NWC; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      for (int i = 0; i < G::KPW; ++i) {
        const uint32_t b = G::k_lane(i % G::KPER, w, lane) + G::k_step(i);
        EXPECT(b % 16 == 0 && b < (uint32_t)tile, "D=%d NWC=%d K piece %d lane %d: offset %u\n", D, NWC, i, lane, b);
        if (b < (uint32_t)tile) ++k[b / 16];
      }
      for (int i = 0; i < G::VPW; ++i) {
        const uint32_t b = G::v_lane(w, lane, 64) + G::v_step(i, 64);
        EXPECT(b % 16 == 0 && b < (uint32_t)tile, "D=%d NWC=%d V piece %d lane %d: offset %u\n", D, NWC, i, lane, b);
        if (b < (uint32_t)tile) ++v[b / 16];
      }
    }
  for (int c = 0; c < tile / 16; ++c) {
    EXPECT(k[c] == 1, "D=%d NWC=%d: K chunk %d copied %d times\n", D, NWC, c, k[c]);
    EXPECT(v[c] == 1, "D=%d NWC=%d: V chunk %d copied %d times\n", D, NWC, c, v[c]);
  }
}

static void fine_bounds(int C) {
  constexpr int D = 128, NWC = 2;
  using G = wf::CopyGeom<D, NWC>;
  const uint32_t CB = 64u * D * 2, region = (uint32_t)C * CB;
  const long long probes[] = {0, 1, C / 2, C - 1, C, C + 1, -1, -2, 2 * (long long)C, 262144, 262144 + 3,
                              (1ll << 20) + 1, INT_MAX, INT_MIN, INT_MIN + 5};
  for (long long p : probes) {
    const int cube = (int)p;
    const bool valid = cube >= 0 && cube < C;
    const uint32_t at = wf::cube_offset(cube, C, CB);
    for (int w = 0; w < NWC; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        for (int i = 0; i < G::KPW + G::VPW; ++i) {
          const bool isk = i < G::KPW;
          const uint32_t lo = isk ? G::k_lane(i % G::KPER, w, lane) : G::v_lane(w, lane, 64);
          const uint32_t st = isk ? G::k_step(i) : G::v_step(i - G::KPW, 64);
          const uint64_t voff = (uint64_t)lo + at;  // per-lane offset (what the range check sees)
          EXPECT(voff < (1ull << 31), "C=%d cube %d: offset %llu does not fit the 32-bit field\n", C, cube,
                 (unsigned long long)voff);
          if (valid) {
            const uint64_t a = voff + st;
            EXPECT(voff < region && a >= (uint64_t)cube * CB && a + 16 <= (uint64_t)(cube + 1) * CB,
                   "C=%d cube %d: access %llu outside its cube\n", C, cube, (unsigned long long)a);
          } else {
            EXPECT(voff >= region, "C=%d bad cube %d: offset %llu inside the region (%u)\n", C, cube,
                   (unsigned long long)voff, region);
          }
        }
      }
  }
}

static void grid_copy(int T, int H, int W) {
  const int nt = (T + 3) / 4, nh = (H + 3) / 4, nw = (W + 3) / 4, C = nt * nh * nw;
  const uint32_t N = (uint32_t)T * H * W;
  for (int cube = -2; cube < C + 2; ++cube) {
    const bool valid = cube >= 0 && cube < C;
    const uint32_t first = wf::cube_first_token(cube, C, nh, nw, H, W, N);
    if (!valid) {
      EXPECT(first == N, "grid %dx%dx%d: bad cube %d starts at token %u, not the end %u\n", T, H, W, cube, first, N);
      continue;
    }
    const int ct = cube / (nw * nh), ch = (cube / nw) % nh, cw = cube % nw;
    for (int i = 0; i < 8; ++i)
      for (int w = 0; w < 2; ++w)
        for (int lane = 0; lane < 64; ++lane) {
          const int slot = 4 * (2 * i + w) + lane / 16;
          const int t = 4 * ct + slot / 16, h = 4 * ch + (slot / 4) % 4, x = 4 * cw + slot % 4;
          const uint64_t off = wf::grid_k_offset(first, i, w, lane, H, W);
          EXPECT(off < (1ull << 31), "grid %dx%dx%d cube %d: offset %llu does not fit\n", T, H, W, cube,
                 (unsigned long long)off);
          const uint64_t voff = wf::grid_v_offset(first, i, w, lane, H, W, T - 4 * ct, H - 4 * ch, W - 4 * cw,
                                                   N * 256u);
          EXPECT((uint64_t)wf::grid_row_part(first, i, w, H, W) + wf::grid_lane_part<false>(i % 2, w, lane) == off,
                 "grid %dx%dx%d cube %d piece %d w %d lane %d: split K offset differs\n", T, H, W, cube, i, w, lane);
          EXPECT((uint64_t)wf::grid_row_part(first, i, w, H, W) + wf::grid_lane_part<true>(i % 2, w, lane) ==
                     wf::grid_v_offset_full(first, i, w, lane, H, W),
                 "grid %dx%dx%d cube %d piece %d w %d lane %d: split V offset differs\n", T, H, W, cube, i, w, lane);
          if (!(t < T && h < H && x < W))
            EXPECT(voff >= (uint64_t)N * 256, "grid %dx%dx%d cube %d: padded V slot %d is read from memory\n", T, H,
                   W, cube, slot);
          if (t < T && h < H && x < W) {  // a real slot: the bytes the cube-ordered copy reads for it
            const uint64_t tok = ((uint64_t)t * H + h) * W + x;
            const uint64_t want = tok * 256 + (uint64_t)wf::Swz<128>::kslot(slot, lane % 16) * 16;
            EXPECT(off == want, "grid %dx%dx%d cube %d piece %d w %d lane %d: %llu, want %llu\n", T, H, W, cube, i,
                   w, lane, (unsigned long long)off, (unsigned long long)want);
            const uint64_t vwant = tok * 256 + (uint64_t)wf::VtrSwz::slot(slot, lane % 16) * 16;
            EXPECT(voff == vwant, "grid %dx%dx%d cube %d V piece %d w %d lane %d\n", T, H, W, cube, i, w, lane);
          }
        }
  }
}

// The V tile as the copy leaves it in LDS (piece 2i + w, lane l -> LDS bytes 16 (64 (2i + w) + l),
// the chunk grid_v_offset fetched), then every transpose read of every P V MFMA.
static void transpose_reads() {
  int row_of[64 * 16], d0_of[64 * 16];  // per 16-byte LDS chunk: its key row and first dim
  for (int i = 0; i < 8; ++i)
    for (int w = 0; w < 2; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t off = wf::grid_v_offset(0, i, w, lane, 4, 4, 4, 4, 4, 64 * 256);  // a 4x4 plane: slot = token
        const int lds = (64 * (2 * i + w) + lane);                    // 16-byte chunk index in LDS
        row_of[lds] = (int)(off / 256);
        d0_of[lds] = (int)(off % 256) / 2;
      }
  for (int ks = 0; ks < 4; ++ks)
    for (int b = 0; b < 4; ++b)
      for (int r = 0; r < 2; ++r) {
        int row[64], d0[64];
        bool bank_used[2][64] = {};
        for (int L = 0; L < 64; ++L) {
          const uint32_t a = wf::VtrSwz::offset(wf::VtrSwz::lane_base(L), ks, b, r);
          EXPECT(a % 8 == 0 && a + 8 <= 64 * 256, "transpose read ks %d b %d r %d lane %d: bad address %u\n", ks, b,
                 r, L, a);
          row[L] = row_of[a / 16];
          d0[L] = d0_of[a / 16] + (int)(a % 16) / 2;
          for (int x = 0; x < 2; ++x) {
            const int bank = (int)(a / 4 + x) % 64;
            EXPECT(!bank_used[L / 32][bank], "transpose read ks %d b %d r %d: bank %d twice in a half wave\n", ks, b,
                   r, bank);
            bank_used[L / 32][bank] = true;
          }
        }
        for (int L = 0; L < 64; ++L) {  // lane L = 16 g + i receives element i % 4 of lanes 16 g + 4 e + i / 4
          const int g = L / 16, i = L % 16, j = L % 32, h = L / 32;
          for (int e = 0; e < 4; ++e) {
            const int src = 16 * g + 4 * e + i / 4;
            const int key = row[src], d = d0[src] + i % 4;
            const int want_key = 16 * ks + 8 * r + 4 * h + e, want_d = 32 * b + j;  // t = 4 r + e
            EXPECT(key == want_key && d == want_d,
                   "transpose read ks %d b %d r %d lane %d element %d: (key %d, d %d), want (%d, %d)\n", ks, b, r, L,
                   e, key, d, want_key, want_d);
          }
        }
      }
}

// The block-coordinate division by multiply-high (div_magic) is exact for every block index
// below 4096 and divisor up to 4096 (and a sample of larger divisors), and block coordinates
// computed with it give cube_first_token's first tokens.
static void magic_division() {
  for (uint32_t d = 1; d <= 4096; ++d) {
    const uint32_t m = wf::div_magic(d);
    for (uint32_t n = 0; n < 4096; ++n)
      EXPECT(wf::div_by_magic(n, m) == n / d, "div_by_magic(%u, magic(%u)) = %u, want %u\n", n, d,
             wf::div_by_magic(n, m), n / d);
  }
  for (uint32_t d = 4097; d < (1u << 20); d += 997) {
    const uint32_t m = wf::div_magic(d);
    for (uint32_t n = 0; n < 4096; n += 7) EXPECT(wf::div_by_magic(n, m) == n / d, "large divisor %u\n", d);
  }
  const int grids[][3] = {{1, 1, 1}, {5, 6, 7}, {21, 30, 52}, {21, 45, 80}, {13, 6, 21}, {64, 64, 64}};
  for (const auto& gr : grids) {
    const int T = gr[0], H = gr[1], W = gr[2];
    const int nh = (H + 3) / 4, nw = (W + 3) / 4, C = (T + 3) / 4 * nh * nw;
    const uint32_t mhw = wf::div_magic((uint32_t)(nh * nw)), mw = wf::div_magic((uint32_t)nw);
    for (int c = 0; c < C; ++c) {
      const int ct = (int)wf::div_by_magic((uint32_t)c, mhw), r = c - ct * nh * nw;
      const int ch = (int)wf::div_by_magic((uint32_t)r, mw), cw = r - ch * nw;
      EXPECT(wf::cube_first_token_at(ct, ch, cw, H, W) == wf::cube_first_token(c, C, nh, nw, H, W, T * H * W),
             "grid %dx%dx%d cube %d: first token differs\n", T, H, W, c);
    }
  }
}

// second_half_padded against the slot layout itself, for both block shapes and every extent of a
// block along each axis (an edge block's 1 .. B-1 tokens, or a whole one).
template <int BT, int BH, int BW>
static void half_padding() {
  for (int lt = 1; lt <= BT + 2; ++lt)
    for (int lh = 1; lh <= BH + 2; ++lh)
      for (int lw = 1; lw <= BW + 2; ++lw) {
        bool all = true;
        for (int s = 32; s < 64; ++s)
          if (s / (BH * BW) < lt && (s / BW) % BH < lh && s % BW < lw) all = false;
        const bool got = wf::second_half_padded<BT, BH, BW>(lt, lh);
        EXPECT(got == all, "block %dx%dx%d extents %d,%d,%d: %d, want %d\n", BT, BH, BW, lt, lh, lw, (int)got, (int)all);
      }
}

int main() {
  half_padding<4, 4, 4>();
  half_padding<1, 8, 8>();
  magic_division();
  transpose_reads();
  coverage<128, 2>();
  coverage<128, 4>();
  coverage<64, 4>();
  for (int C : {1, 8, 27, 624, 1200, 1296, 1440, 4096}) fine_bounds(C);
  const int grids[][3] = {{1, 1, 1}, {4, 4, 4}, {5, 6, 7}, {9, 10, 11}, {21, 30, 52}, {21, 45, 80}, {13, 6, 21}};
  for (const auto& gr : grids) grid_copy(gr[0], gr[1], gr[2]);
  if (fails) {
    printf("%d failures\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
