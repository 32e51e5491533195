// Host check of the copy arithmetic the kernels use (wf_tiles.hpp, built here with g++):
//  * every K / V^T tile copy covers each 16-byte chunk of the tile exactly once;
//  * in the fine stage a key cube inside [0, C) is read only from its own 16 KiB, and an
//    index outside [0, C) -- any int, including ones whose byte offset would wrap 32 bits --
//    gets a per-lane offset at or past the end of the head's region, which the buffer
//    descriptor's range check turns into zeros.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <climits>
#include <vector>

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

int main() {
  coverage<128, 2>();
  coverage<128, 4>();
  coverage<64, 4>();
  for (int C : {1, 8, 27, 624, 1200, 1296, 1440, 4096}) fine_bounds(C);
  if (fails) {
    printf("%d failures\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
