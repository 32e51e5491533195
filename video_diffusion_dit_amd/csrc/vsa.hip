// Video Sparse Attention (VSA) on gfx950: cube gather and pooling, coarse
// cube scores, per-cube top-k and fine block-sparse attention.
//
// Operation: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "VSA
// selects cubes": pad the T x H x W grid to multiples of 4, cut it into 4x4x4
// cubes of 64 tokens, score cube-mean queries against cube-mean keys, keep the
// top-k key cubes of every query cube, then run token-level attention of each
// query cube over those cubes only.  Section "Roofline analysis set the 3.35
// ms target" counts one output tile per (query cube, head).
#include <type_traits>

#include "wf_attn.h"
#include "wf_device.hpp"
#include "wf_grid.hpp"
#include "wf_launch.hpp"
#include "wf_rope.hpp"

namespace wf {

static_assert(kSoftmaxGuarded == WF_SOFTMAX_GUARDED && kSoftmaxRunningMax == WF_SOFTMAX_RUNNING_MAX &&
                  kSoftmaxFixedFirst == WF_SOFTMAX_FIXED_FIRST_TILE,
              "softmax policy numbers of the C ABI and the kernels");

// Blocks of 64 tokens the gather and the fine stage work on: VSA's 4x4x4 cubes
// ("VSA selects cubes"), and 1x8x8 slabs for sliding-tile attention, whose
// 6x8x8 tiles are six slabs stacked along t.  Slot s of a block is row-major:
// (s / (BH*BW), s / BW % BH, s % BW).
template <int BT_, int BH_, int BW_>
struct Block {
  static constexpr int BT = BT_, BH = BH_, BW = BW_;
  static_assert(BT * BH * BW == 64, "a block is 64 tokens");
};
using Cube = Block<4, 4, 4>;
using Slab = Block<1, 8, 8>;

// The block grid of a T x H x W token grid (each axis padded up to a whole
// number of blocks).  Cs: the block count rounded up to a multiple of 32, the
// row stride of the coarse scores and of the transposed cube means of V.
// mnw, mnhw: div_magic of nw and nh * nw, so that block coordinates cost two multiply-highs.
struct Grid3 {
  int T, H, W, nt, nh, nw, C, Cs;
  uint32_t mnw, mnhw;
};

template <class BLK>
static Grid3 make_grid(int T, int H, int W) {
  Grid3 g{T, H, W, (T + BLK::BT - 1) / BLK::BT, (H + BLK::BH - 1) / BLK::BH, (W + BLK::BW - 1) / BLK::BW, 0, 0, 0, 0};
  g.C = g.nt * g.nh * g.nw;
  g.Cs = (g.C + 31) / 32 * 32;
  g.mnw = div_magic((uint32_t)g.nw);
  g.mnhw = div_magic((uint32_t)(g.nh * g.nw));
  return g;
}

// Blocks of 32 cubes of the stored cube means of Q and K: the scores' 128-wide
// tiles cover C rounded up to 128 (rows and columns).
__host__ __device__ constexpr int mean_blocks(int C) { return (C + 127) / 128 * 4; }

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element offset of (part, head, key cube, head dim) in the cube means of V,
// stored in the lane order of the coarse-branch MFMA's A operand so that one
// load of a wavefront reads 1 KiB contiguously: [part hi/lo][bh][key step of
// 16][dim block of 32][lane 0..63][8 key cubes], lane = dim % 32 + 32 * (key % 16 / 8).
__device__ __forceinline__ long vbar_index(int part, int bh, int BH, int Cs, int key, int d) {
  const int lane = d % 32 + 32 * ((key % 16) / 8);
  return ((((long)part * BH + bh) * (Cs / 16) + key / 16) * 4 + d / 32) * 512 + lane * 8 + key % 8;
}

// Element offset of (head, cube, head dim, part) in the cube means of Q or K,
// each fp32 mean stored as three bf16 parts (mean_split), in the operand lane
// order of the coarse scores' MFMAs (wf_vsa_scores) so that each of a
// wavefront's operand loads reads 1 KiB contiguously: [bh][block of 32
// cubes][d step of 16][part hi/mid/lo][lane 0..63][8], lane = cube % 32 +
// 32 * (d % 16 / 8).  nrb blocks of 32 cubes per head (rows past C are never
// written; their scores are discarded).
__device__ __forceinline__ long mean_index(int bh, int nrb, int D, int c, int d, int part) {
  const int lane = c % 32 + 32 * ((d % 16) / 8);
  return (((((long)bh * nrb + c / 32) * (D / 16) + d / 16) * 3 + part) * 64 + lane) * 8 + d % 8;
}

// An fp32 value as three bf16 parts, each rounded to nearest: hi = bf16(x),
// mid = bf16(x - hi), lo = bf16(x - hi - mid).  Each difference is exact in
// fp32 and the last one has at most 8 significant bits, so hi + mid + lo == x
// exactly for every normal x (bf16 keeps fp32's exponent range).
struct MeanSplit {
  uint16_t part[3];
};
__device__ __forceinline__ MeanSplit mean_split(float x) {
  const __bf16 h = (__bf16)x;
  const float r1 = x - (float)h;
  const __bf16 m = (__bf16)r1;
  const __bf16 l = (__bf16)(r1 - (float)m);
  return {{__builtin_bit_cast(uint16_t, h), __builtin_bit_cast(uint16_t, m), __builtin_bit_cast(uint16_t, l)}};
}

// Token of slot s in block (ct, ch, cw), or -1 for a padded slot.
template <class BLK>
__device__ __forceinline__ int slot_token(const Grid3& g, int ct, int ch, int cw, int s) {
  const int t = ct * BLK::BT + s / (BLK::BH * BLK::BW), h = ch * BLK::BH + (s / BLK::BW) % BLK::BH,
            w = cw * BLK::BW + s % BLK::BW;
  return (t < g.T && h < g.H && w < g.W) ? (t * g.H + h) * g.W + w : -1;
}

// Block coordinates of block c (0 <= c < C <= 4096; any other c gives some coordinates, which
// callers do not use to address memory).
__device__ __forceinline__ void cube_coords(const Grid3& g, int c, int& ct, int& ch, int& cw) {
  ct = (int)div_by_magic((uint32_t)c, g.mnhw);
  const int r = c - ct * g.nh * g.nw;
  ch = (int)div_by_magic((uint32_t)r, g.mnw);
  cw = r - ch * g.nw;
}

// Where key block `cube` lies: how far it extends inside the grid along t, h and w (the block's
// full size for an interior block) and its first token, or n_tokens for an index outside [0, C).
struct BlockAt {
  uint32_t first;
  int lt, lh, lw;
};
template <class BLK>
__device__ __forceinline__ BlockAt block_at(const Grid3& g, int cube, uint32_t n_tokens) {
  int bt, bh, bw;
  cube_coords(g, cube, bt, bh, bw);
  BlockAt a;
  a.lt = g.T - BLK::BT * bt;
  a.lh = g.H - BLK::BH * bh;
  a.lw = g.W - BLK::BW * bw;
  a.first = (uint32_t)cube < (uint32_t)g.C ? block_first_token<BLK::BT, BLK::BH, BLK::BW>(bt, bh, bw, g.H, g.W)
                                           : n_tokens;
  return a;
}

// Whether keys (or query slots) 32..63 of block `a` are all padding: the second score block of a
// key tile (its probabilities are zero) or the second wavefront's query rows.
template <class BLK>
__device__ __forceinline__ bool upper_half_padded(const BlockAt& a) {
  return second_half_padded<BLK::BT, BLK::BH, BLK::BW>(a.lt, a.lh);
}

// ---------------------------------------------------------------- gather + pool
// One workgroup per (bh, block).  Writes Qc, Kc [BH][C][64][D] (padded slots
// zero), Vct [BH][C][D][64] (slots in perm16 order) and, with POOL, the fp32
// means of Q and K over the block's real tokens, each as three bf16 parts in
// the scores' operand order (mean_split, mean_index), and the fp32 mean of V split
// into two bf16 parts, hi = bf16(mean) and lo = bf16(mean - hi), at key cube c
// of the operand-ordered means (vbar_index; key cubes C..Cs-1 are zeroed, so
// the coarse-branch product may run over whole 32-wide steps).  With ROPE, Q
// and K are rotated by the 3D RoPE (wf_rope.hpp) on the way in, so everything
// downstream (cube means, scores, the fine stage) sees the rotated vectors;
// the cube's 4 t, 4 h and 4 w coordinates need one table of 4*(t2+h2+w2)
// (cos, sin) pairs, one fp64 sincos per thread.  ROPE is the rotation's
// precision (32 or 64), 0 for none.  BLK is the block shape (VSA's cubes, or
// sliding-tile attention's slabs, which need no means).  Q, K, V are read and
// the copies written with the streaming (non-temporal) policy: each byte is
// touched once here (3% faster than the default policy at 480p).  OUT selects
// what else is written: the cube-ordered Qc and Kc (kOutQK), Vct (kOutVt) and,
// with POOL, the mean of V (kOutVbar); V is read only for the last two.  The
// one-call path's fine stage reads Q and K (and, up to some top-k, V) from the
// token grid, so there the gather writes only the means (and Vct where V is
// not read from the grid, the mean of V where the coarse branch needs it).
constexpr int kOutQK = 1, kOutVt = 2, kOutVbar = 4, kOutAll = 7;
template <int D, int ROPE, class BLK = Cube, bool POOL = true, int OUT = kOutAll>
__global__ void __launch_bounds__(256) wf_vsa_gather(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qc, uint16_t* __restrict__ kc, uint16_t* __restrict__ vct,
    uint16_t* __restrict__ qbar, uint16_t* __restrict__ kbar, uint16_t* __restrict__ vbt, Grid3 g,
    double theta) {
  static_assert(ROPE == 0 || (BLK::BT == 4 && BLK::BH == 4 && BLK::BW == 4), "RoPE is fused for cubes only");
  constexpr int ROWCH = D / 8;            // 16-byte chunks per row
  constexpr int RSTEP = 256 / ROWCH;      // rows covered by one pass of the workgroup
  constexpr int VSTR = D + 2;
  constexpr RopeSplit sp = rope_split(D);
  constexpr int NTAB = ROPE ? 4 * (sp.t2 + sp.h2 + sp.w2) : 1;
  using CS = RopeCS<ROPE == 64 ? 64 : 32>;
  __shared__ float red[POOL ? RSTEP : 1][D];
  __shared__ uint16_t vtile[(OUT & kOutVt) ? 64 * VSTR : 1];
  __shared__ CS tab[NTAB];
  const int tid = threadIdx.x, c16 = tid % ROWCH, r0 = tid / ROWCH;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.C, c = item % g.C;
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
  if constexpr (ROPE != 0) {  // [4 t][t2] then [4 h][h2] then [4 w][w2]
    for (int e = tid; e < NTAB; e += 256) {
      if (e < 4 * sp.t2)
        tab[e] = rope_cs<CS>(4 * ct + e / sp.t2, rope_freq(e % sp.t2, 2 * sp.t2, theta));
      else if (e < 4 * (sp.t2 + sp.h2))
        tab[e] = rope_cs<CS>(4 * ch + (e - 4 * sp.t2) / sp.h2, rope_freq((e - 4 * sp.t2) % sp.h2, 2 * sp.h2, theta));
      else
        tab[e] = rope_cs<CS>(4 * cw + (e - 4 * (sp.t2 + sp.h2)) / sp.w2,
                             rope_freq((e - 4 * (sp.t2 + sp.h2)) % sp.w2, 2 * sp.w2, theta));
    }
    __syncthreads();
  }
  const long N = (long)g.T * g.H * g.W;
  const long cube_row0 = ((long)bh * g.C + c) * 64;
  const int count = min(BLK::BT, g.T - BLK::BT * ct) * min(BLK::BH, g.H - BLK::BH * ch) *
                    min(BLK::BW, g.W - BLK::BW * cw);

  for (int which = 0; which < ((OUT & (kOutVt | kOutVbar)) ? 3 : 2); ++which) {
    const uint16_t* src = (which == 0 ? q : which == 1 ? k : v) + (long)bh * N * D;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 64 / RSTEP; ++i) {
      const int s = r0 + i * RSTEP;
      const int tok = slot_token<BLK>(g, ct, ch, cw, s);
      uint4 u = make_uint4(0, 0, 0, 0);
      if (tok >= 0)
        u = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (long)tok * D + c16 * 8)));
      if constexpr (ROPE != 0) {
        if (which < 2 && tok >= 0) {
          const int st = s >> 4, sh = (s >> 2) & 3, sw = s & 3;
          u = rope_rotate_chunk(u, c16 * 4, [&](int p) {
            return p < sp.t2 ? tab[st * sp.t2 + p]
                 : p < sp.t2 + sp.h2 ? tab[4 * sp.t2 + sh * sp.h2 + (p - sp.t2)]
                                     : tab[4 * (sp.t2 + sp.h2) + sw * sp.w2 + (p - sp.t2 - sp.h2)];
          });
        }
      }
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&u);
      if (which < 2) {
        if constexpr ((OUT & kOutQK) != 0) {
          uint16_t* dst = (which == 0 ? qc : kc) + (cube_row0 + s) * D + c16 * 8;
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, u), reinterpret_cast<u32x4*>(dst));
        }
      } else if constexpr ((OUT & kOutVt) != 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) vtile[s * VSTR + c16 * 8 + t] = e[t];
      }
      if constexpr (POOL) {
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += __uint_as_float((uint32_t)e[t] << 16);
      }
    }
    if constexpr (POOL) {
#pragma unroll
      for (int t = 0; t < 8; ++t) red[r0][c16 * 8 + t] = acc[t];
      __syncthreads();
      if (tid < D) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RSTEP; ++r) sum += red[r][tid];
        const float mean = sum / (float)count;
        if (which < 2) {
          const MeanSplit ms = mean_split(mean);
#pragma unroll
          for (int p = 0; p < 3; ++p)
            (which == 0 ? qbar : kbar)[mean_index(bh, mean_blocks(g.C), D, c, tid, p)] = ms.part[p];
        } else if constexpr ((OUT & kOutVbar) != 0) {
          static_assert(D == 128, "four 32-wide head-dim blocks");
          const int BH = gridDim.x / g.C;  // gridDim.x = BH * C
          const __bf16 h16 = (__bf16)mean;
          vbt[vbar_index(0, bh, BH, g.Cs, c, tid)] = __builtin_bit_cast(uint16_t, h16);
          vbt[vbar_index(1, bh, BH, g.Cs, c, tid)] = __builtin_bit_cast(uint16_t, (__bf16)(mean - (float)h16));
          for (int x = g.C + c; x < g.Cs; x += g.C)
            vbt[vbar_index(0, bh, BH, g.Cs, x, tid)] = vbt[vbar_index(1, bh, BH, g.Cs, x, tid)] = 0;
        }
      }
    }
    __syncthreads();
    if ((OUT & kOutVt) != 0 && which == 2) {
      uint16_t* dst = vct + ((long)bh * g.C + c) * D * 64;
      for (int id = tid; id < D * 8; id += 256) {
        const int d = id / 8, pc = id % 8;
        uint16_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = vtile[perm16(pc * 8 + t) * VSTR + d];
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(e),
                                    reinterpret_cast<u32x4*>(dst + d * 64 + pc * 8));
      }
    }
  }
}

// ---------------------------------------------------------------- coarse scores
// S[bh][c][c'] = scale * sum_d Qbar[c][d] Kbar[c'][d] to fp32 accuracy, from
// the three-part bf16 split of each fp32 mean (x = hi + mid + lo exactly,
// mean_split) on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16): the six
// partial products lo*hi, mid*mid, hi*lo, mid*hi, hi*mid, hi*hi, smallest
// first, accumulated in fp32.  The three dropped ones (mid*lo, lo*mid, lo*lo)
// are each below 2^-23 of |Qbar_d Kbar_d|, the order of one fp32 rounding; the
// six take 6 x 32 matrix-core cycles per 16 d where fp32 MFMAs take 8 x 64.
// One workgroup (4 wavefronts) per 128x128 tile of S, a 64x64 tile (2x2
// blocks of 32x32) per wavefront, so each operand row a wavefront loads feeds
// two blocks.  Lane (j, h) takes d = 16 u + 8 h .. + 7 at step u for both
// operands, 16 bytes of one part of one row, read straight from memory (L2),
// no LDS; the means are stored in this lane order (mean_index), so every load
// of a wavefront reads 1 KiB contiguously (8 cache lines, where row-major
// means made each load touch 32).  Workgroups are renumbered per XCD
// (xcd_remap) so each XCD's L2 holds the means of few heads.  s has row stride
// Cs and -inf in columns C..Cs-1; s_user (optional) gets the same scores with
// row stride C.
template <int D>
__global__ void __launch_bounds__(256) wf_vsa_scores(const uint16_t* __restrict__ qbar,
                                                     const uint16_t* __restrict__ kbar,
                                                     float* __restrict__ s, float* __restrict__ s_user,
                                                     int C, int Cs, int ntr, int ntc, float scale) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, j = lane % 32,
            h = lane / 32;
  const int per_head = ntr * ntc, nrb = 4 * ntr;  // ntr = ntc = mean_blocks(C) / 4
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / per_head, rem = item % per_head;
  // workgroup tile 128 x 128, wavefront tile 64 x 64 = 2 x 2 blocks of 32 x 32
  const int r0 = (rem / ntc) * 128 + (wave >> 1) * 64, c0 = (rem % ntc) * 128 + (wave & 1) * 64;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    arow[x] = qbar + mean_index(bh, nrb, D, r0 + 32 * x, 0, 0) + lane * 8;
    brow[x] = kbar + mean_index(bh, nrb, D, c0 + 32 * x, 0, 0) + lane * 8;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.f;
  // (A part, B part) of the six products, smallest first: 0 = hi, 1 = mid, 2 = lo
  constexpr int PA[6] = {2, 1, 0, 1, 0, 0}, PB[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll 2
  for (int u = 0; u < D / 16; ++u) {
    bf16x8 a[2][3], b[2][3];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        a[x][p] = as_bf16x8(*reinterpret_cast<const uint4*>(arow[x] + (u * 3 + p) * 512));
        b[x][p] = as_bf16x8(*reinterpret_cast<const uint4*>(brow[x] + (u * 3 + p) * 512));
      }
#pragma unroll
    for (int t = 0; t < 6; ++t)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x][PA[t]], b[y][PB[t]], acc[x][y], 0, 0, 0);
  }
  // block (x, y): lane (j, h) holds S[r0 + 32x + 8*(i/4) + 4h + i%4][c0 + 32y + j]
  float* out = s + (long)bh * C * Cs;
  float* user = s_user ? s_user + (long)bh * C * C : nullptr;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int cc = c0 + 32 * y + j;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = r0 + 32 * x + 8 * (i / 4) + 4 * h + i % 4;
        if (r >= C) continue;
        const float val = acc[x][y][i] * scale;
        if (cc < Cs) out[(long)r * Cs + cc] = cc < C ? val : -INFINITY;
        if (user && cc < C) user[(long)r * C + cc] = val;
      }
    }
}

// ---------------------------------------------------------------- top-k
// One wavefront per score row.  Lane L holds candidates c' = e*64 + L.  The
// k-th largest order key is found bit by bit (count of keys >= candidate via
// ballots); keys above it are all kept, keys equal to it are kept in
// ascending c' order until k are chosen.  Output is ascending.  The wavefront
// also records the row's softmax statistics for the coarse-branch output:
// stat[row] = (log2(e) * max_c' S, 1 / sum_c' 2^(log2(e) S - that)).
template <int E>
__global__ void __launch_bounds__(256) wf_vsa_topk(const float* __restrict__ s,
                                                   int* __restrict__ idx, float2* __restrict__ stat,
                                                   long rows, int C, int Cs, int k) {
  const int lane = threadIdx.x % 64;
  const long row = (long)blockIdx.x * 4 + threadIdx.x / 64;
  if (row >= rows) return;
  const float* sr = s + row * Cs;
  uint32_t key[E];
  float val[E];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int cc = e * 64 + lane;
    val[e] = cc < C ? sr[cc] : -INFINITY;
    key[e] = cc < C ? order_key(val[e]) : 0u;
    mx = fmaxf(mx, val[e]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float ml = mx * kLog2e;
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(val[e], kLog2e, -ml));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) stat[row] = make_float2(ml, 1.f / sum);
  // thr ends as the k-th largest key, or -- when some candidate has exactly k keys at or above
  // it, which usually happens long before bit 0 -- as that candidate minus one, so that the keys
  // above thr are exactly the k largest and no tie is left to resolve (the same set either way)
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
    if (cnt == k) {
      thr = cand - 1u;
      break;
    }
    if (cnt > k) thr = cand;
  }
  int ngt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) ngt += __popcll(__ballot(key[e] > thr));
  const int need = k - ngt;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* out = idx + row * k;
  int pos = 0, ties = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = key[e] == thr;
    const uint64_t beq = __ballot(eq);
    const bool sel = key[e] > thr || (eq && ties + __popcll(beq & below) < need);
    const uint64_t bsel = __ballot(sel);
    const int at = pos + __popcll(bsel & below);
    if (sel && at < k) out[at] = e * 64 + lane;
    pos += __popcll(bsel);
    ties += __popcll(beq);
  }
}

// ---------------------------------------------------------------- coarse-branch output
// Oc[bh][c] = sum_c' softmax_c'(S[c][c']) Vbar[c'], the cube-level attention
// of the coarse stage, from the fp32 scores and the row statistics the top-k
// kernel recorded (so P is final: no running max, no rescale).  One workgroup
// per (bh, 32 query cubes); its four wavefronts take interleaved steps of 16
// key cubes (wavefront w: steps w, w+4, ...), each accumulating all D head
// dims, and the four partial sums are added through LDS at the end:
//   Oc^T (D x 32) = Vbar^T (D x Cs) . P^T (Cs x 32), MFMA 32x32x16 bf16,
// with both operands split into bf16 hi and lo parts and the three products
// hi.hi + lo.hi + hi.lo summed in fp32: an error near fp32's, where bf16
// operands alone would carry Vbar's rounding straight into Oc (the softmax
// over cubes is usually dominated by one cube).  Each lane builds its B
// operand straight from one score row (one query cube, 8 consecutive key
// cubes) and reads its A operands (8 consecutive key cubes of one head dim)
// from the operand-ordered means, 1 KiB per wavefront and load; both operands
// index key cubes the same way, so the product pairs them correctly.  The next step's operands are loaded before the
// current step's products.  Padded key columns hold -inf scores and zero
// means, so they add nothing.
template <int D>
struct CoarseStep {
  float4 x[2];          // 8 scores of this lane's query cube
  uint4 a[2 * (D / 32)];  // Vbar^T hi (blocks 0..DB-1), then lo
};

template <int D>
__device__ __forceinline__ void coarse_load(CoarseStep<D>& st, const float* srow, const uint16_t* va,
                                            long lo_off, int t) {
  constexpr int DB = D / 32;
  st.x[0] = *reinterpret_cast<const float4*>(srow + t * 16);
  st.x[1] = *reinterpret_cast<const float4*>(srow + t * 16 + 4);
#pragma unroll
  for (int u = 0; u < 2 * DB; ++u)
    st.a[u] = *reinterpret_cast<const uint4*>(va + (u / DB) * lo_off + ((long)t * DB + u % DB) * 512);
}

template <int D>
__global__ void __launch_bounds__(256) wf_vsa_coarse_out(const float* __restrict__ s,
                                                         const float2* __restrict__ stat,
                                                         const uint16_t* __restrict__ vbt,
                                                         float* __restrict__ oc, int C, int Cs,
                                                         int rblocks) {
  constexpr int DB = D / 32;
  __shared__ float part[4][DB][16][64];  // per wavefront: DB accumulator blocks, register-major
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64,
            j = lane % 32, half = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / rblocks, rb = item % rblocks;
  const int r = rb * 32 + j, rr = min(r, C - 1);
  const float2 st = stat[(long)bh * C + rr];
  const float* srow = s + ((long)bh * C + rr) * Cs + half * 8;
  const int BH = gridDim.x / rblocks;  // gridDim.x = BH * rblocks
  const uint16_t* va = vbt + vbar_index(0, bh, BH, Cs, 0, 0) + lane * 8;  // hi part, step 0, block 0
  const long lo_off = (long)BH * D * Cs;                                    // lo part follows hi
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  const int nsteps = Cs / 16;
  CoarseStep<D> cur, nxt;
  if (wave < nsteps) coarse_load<D>(cur, srow, va, lo_off, wave);
  for (int t = wave; t < nsteps; t += 4) {
    const int tn = t + 4 < nsteps ? t + 4 : t;  // past the end: reload the current step (in bounds)
    coarse_load<D>(nxt, srow, va, lo_off, tn);
    const float xs[8] = {cur.x[0].x, cur.x[0].y, cur.x[0].z, cur.x[0].w,
                         cur.x[1].x, cur.x[1].y, cur.x[1].z, cur.x[1].w};
    f32x8 pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[i], kLog2e, -st.x)) * st.y;
    const bf16x8 ph = __builtin_convertvector(pf, bf16x8);
    const bf16x8 pl = __builtin_convertvector(pf - __builtin_convertvector(ph, f32x8), bf16x8);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.a[DB + b]), ph, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.a[b]), pl, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.a[b]), ph, acc[b], 0, 0, 0);
    }
    cur = nxt;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][b][i][lane] = acc[b][i];
  __syncthreads();
  // wavefront w adds up accumulator block w (D = 128: one block each) and stores it
  for (int b = wave; b < DB; b += 4) {
    float o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o[i] = (part[0][b][i][lane] + part[1][b][i][lane]) + (part[2][b][i][lane] + part[3][b][i][lane]);
    if (r < C) {
      float* orow = oc + ((long)bh * C + r) * D + b * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(orow + q * 8 + half * 4) = make_float4(o[q * 4], o[q * 4 + 1], o[q * 4 + 2], o[q * 4 + 3]);
    }
  }
}

// Gate rows and the query cube's coarse output for the gated merge, loaded
// into registers ahead of the epilogue (lane L takes 4 head dims, chunk L % 32,
// of rows 2i + L/32 of its wavefront's 32 query slots).  Padded slots load
// the cube's first row instead (read, never used), so every lane issues the
// same loads.
struct GatePre {
  uint2 g[16];
  float4 c4;
};

template <int D, class BLK>
__device__ __forceinline__ void gate_prefetch(GatePre& gp, const Grid3& g, int ct, int ch, int cw, int wave,
                                              int lane, long head_row0, const uint16_t* __restrict__ gate,
                                              const float* __restrict__ ocube) {
  const int c = lane % 32;
  const int tok0 = slot_token<BLK>(g, ct, ch, cw, 0);  // slot 0 is always a real token
  gp.c4 = *reinterpret_cast<const float4*>(ocube + c * 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = slot_token<BLK>(g, ct, ch, cw, wave * 32 + 2 * i + lane / 32);
    gp.g[i] = *reinterpret_cast<const uint2*>(gate + (head_row0 + (tok >= 0 ? tok : tok0)) * D + c * 4);
  }
}

// Fine-stage epilogue: the normalised output rows of a wavefront go through
// its own LDS slot (32 rows x D fp32 = 16 KiB, the K or V slot, free once the
// sweep is done), so that global stores cover two whole token rows per
// instruction instead of 16 bytes of 32 different rows.  In LDS, row r's
// 16-byte chunk c sits at chunk c ^ (r % 32), which keeps both the scattered
// writes and the row reads free of bank conflicts.  With GATED the merge
// O = O_fine + gate * Oc is applied on the way out, from the gate rows
// prefetched into gp.
template <int D, bool GATED, class BLK>
__device__ __forceinline__ void fine_epilogue(const f32x16* o, float inv, char* slot_lds, int j, int half,
                                              const Grid3& g, int ct, int ch, int cw, int wave, long head_row0,
                                              float* __restrict__ out, const GatePre& gp) {
  constexpr int DB = D / 32, CH = D / 4;  // 16-byte chunks per row
  static_assert(CH == 32, "row swizzle assumes 32 chunks per row");
  float* lds = reinterpret_cast<float*>(slot_lds);
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int c = (b * 32 + rq * 8 + half * 4) / 4;
      *reinterpret_cast<float4*>(lds + j * D + ((c ^ j) * 4)) =
          make_float4(o[b][rq * 4] * inv, o[b][rq * 4 + 1] * inv, o[b][rq * 4 + 2] * inv, o[b][rq * 4 + 3] * inv);
    }
  asm volatile("" ::: "memory");  // this wavefront's LDS writes precede its reads (LDS keeps wave order)
  const int lane = half * 32 + j, c = lane % 32;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + lane / 32;  // row inside this wavefront's 32
    const int tok = slot_token<BLK>(g, ct, ch, cw, wave * 32 + r);
    float4 v = *reinterpret_cast<const float4*>(lds + r * D + ((c ^ r) * 4));
    if (tok >= 0) {
      const long row = head_row0 + tok;
      if constexpr (GATED) {
        const uint2 g2 = gp.g[i];
        v.x = __builtin_fmaf(__uint_as_float(g2.x << 16), gp.c4.x, v.x);
        v.y = __builtin_fmaf(__uint_as_float(g2.x & 0xFFFF0000u), gp.c4.y, v.y);
        v.z = __builtin_fmaf(__uint_as_float(g2.y << 16), gp.c4.z, v.z);
        v.w = __builtin_fmaf(__uint_as_float(g2.y & 0xFFFF0000u), gp.c4.w, v.w);
      }
      *reinterpret_cast<float4*>(out + row * D + c * 4) = v;
    }
  }
}

// ---------------------------------------------------------------- grid-order K copy
// Copy of key cube `cube` of one head's K straight from the token grid (K [N][D], tokens in
// row-major (t, h, w) order), for the one-call path, which skips the cube-ordered copy of K.
// The LDS tile is the one cube_copy writes: piece i of wavefront w holds cube slots
// 4 (2i + w) .. +3, i.e. slot row dt = (2i + w) / 4, dh = (2i + w) % 4, dw = lane / 16, 16 lanes
// of 16 bytes per token row with the chunk swizzle of Swz.  A slot outside the grid reads some
// other row of the head, or zeros past its end (range check); those keys are masked before the
// softmax.  A cube index outside [0, C) starts at the head's end and reads zeros.
template <int D>
__device__ __forceinline__ void grid_k_copy(const uint16_t* khead, uint32_t head_bytes, char* kdst, const BlockAt& at,
                                            const Grid3& g, int w, int lane) {
  static_assert(D == 128, "16 chunks of 16 bytes per row");
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(khead, head_bytes);
  const uint32_t lp[2] = {grid_lane_part<false>(0, w, lane), grid_lane_part<false>(1, w, lane)};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(kdst + (i * 2 + w) * 1024), 16,
                                             (int)(grid_row_part(at.first, i, w, g.H, g.W) + lp[i % 2]), 0, 0, 0);
}

// The same for a V tile from the token grid's V, laid out for transpose reads (VtrSwz): the P V
// operands are then read as V^T without a transposed copy of V.  Slots outside the grid read
// zeros (grid_v_offset), as in the cube-ordered copy.
template <int D>
__device__ __forceinline__ void grid_v_copy(const uint16_t* vhead, uint32_t head_bytes, char* vdst, const BlockAt& at,
                                            const Grid3& g, int w, int lane) {
  static_assert(D == 128, "16 chunks of 16 bytes per row");
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vhead, head_bytes);
  if (at.lt >= 4 && at.lh >= 4 && at.lw >= 4) {  // an interior cube: every slot is a token
    const uint32_t lp[2] = {grid_lane_part<true>(0, w, lane), grid_lane_part<true>(1, w, lane)};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(vdst + (i * 2 + w) * 1024), 16,
                                               (int)(grid_row_part(at.first, i, w, g.H, g.W) + lp[i % 2]), 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_ptr)(vdst + (i * 2 + w) * 1024), 16,
          (int)grid_v_offset(at.first, i, w, lane, g.H, g.W, at.lt, at.lh, at.lw, head_bytes), 0, 0, 0);
  }
}

// ---------------------------------------------------------------- fine stage
// P V of the previous tile interleaved with the probabilities of the current
// one (p = 2^(s*sl2 - m) in bf16, as tile_probs): step i computes probability
// pair i (two exp2, one convert) and adds it to this lane's sum, then issues
// P V MFMA i, whose V^T operand was read kRingPF steps ahead.  The softmax's
// VALU work thus issues while the matrix pipe runs.  Registers an MFMA reads
// must not be rewritten while it may still read them, so every operand stays
// live until the last MFMA has been issued (the P groups are built once,
// before the first MFMA; each ring slot is refilled at the start of the step
// after the one that consumed it, before any VALU work), and the function
// ends by reading the last MFMA's result, which waits for the matrix pipe to
// drain before any later instruction may reuse those registers.  Returns the
// lane's sum of the new probabilities, summed in tile_probs' order.
//
// Keys 32..63 of an edge block may all be padding (upper_half_padded): their
// probabilities are then zero.  hv (uniform over the wavefront) says the
// previous tile was such a block: its P V pairs 8..15, which would add zeros,
// are skipped by scalar branches, one per step (a single branch between two
// copies of steps 8..15 costs the kernel its register budget); a caller that
// passes a constant false gets no branches.  Each probability pair is pinned
// to its step (an empty asm on the sum it feeds): with branches in the
// sequence the compiler would otherwise sink the pairs that only feed a sum
// past them and bunch them up, away from the MFMAs they are meant to overlap.
template <int D, bool VTR>
__device__ __forceinline__ float pv_with_probs(const char* vt, const bf16x2* p_old, f32x16* o, const f32x16& s0,
                                               const f32x16& s1, float sl2, float m, bf16x2* p_new,
                                               const OperandTable<D, VTR>& tb, bool hv) {
  constexpr int NPV = Pairs<D>::NPV, PF = kRingPF, R = kRing;
  static_assert(NPV == 16 && D == 128, "one probability pair per P V MFMA");
  bf16x8 pg[4];  // B operand of the k-step ks: probabilities 4 ks .. 4 ks + 3
#pragma unroll
  for (int g = 0; g < 4; ++g)
    pg[g] = __builtin_bit_cast(bf16x8, P4{p_old[4 * g], p_old[4 * g + 1], p_old[4 * g + 2], p_old[4 * g + 3]});
  uint4 ring[R];
#pragma unroll
  for (int u = 0; u < PF; ++u) ring[u] = table_operand<D, VTR>(u, vt, nullptr, tb);
  const float nm = -m;
  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  float la = 0.f, lb = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    if (i + PF < NPV) ring[(i + PF) % R] = table_operand<D, VTR>(i + PF, vt, nullptr, tb);
    __builtin_amdgcn_sched_barrier(0);
    const f32x16& sv = i < 8 ? s0 : s1;
    const int r = i % 8;
    p_new[i] = __builtin_convertvector((f32x2){__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * r], sl2, nm)),
                                               __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * r + 1], sl2, nm))},
                                       bf16x2);
    if (i % 2 == 0) {
      la = __builtin_amdgcn_fdot2_f32_bf16(p_new[i], one2, la, false);
      asm volatile("" : "+v"(la));
    } else {
      lb = __builtin_amdgcn_fdot2_f32_bf16(p_new[i], one2, lb, false);
      asm volatile("" : "+v"(lb));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i < 8 || !hv) {
      const int ks = i / 4, b = i % 4;  // mfma_pair's numbering of the P V pairs
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ring[i % R]), pg[ks], o[b], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  auto v4 = [](auto x) __attribute__((always_inline)) { return __builtin_bit_cast(i32x4, x); };
  asm volatile("" ::"v"(v4(pg[0])), "v"(v4(pg[1])), "v"(v4(pg[2])), "v"(v4(pg[3])), "v"(v4(ring[0])),
               "v"(v4(ring[1])), "v"(v4(ring[2])), "v"(v4(ring[3])), "v"(v4(ring[4])));
  __builtin_amdgcn_sched_barrier(0);
  // o[3] is the last MFMA's accumulator (pair 15, or pair 7 with hv): reading it waits for the
  // pipe (0 * o adds nothing to a finite sum; a non-finite O turns the sum into NaN, which only
  // sends the caller to its recompute path)
  return __builtin_fmaf(o[3][15], 0.f, la) + lb;
}

// softmax_tile for tile t with P(t-1) V(t-1) run inside it (pv_with_probs).
// The arithmetic is softmax_tile's, in the same order relative to O: P V of
// tile t-1 is accumulated before O is rescaled for tile t's reference.
template <int D, int SM, bool VTR>
__device__ __forceinline__ void softmax_tile_pv(const char* vt, const bf16x2* p_old, const f32x16& s0,
                                                const f32x16& s1, float sl2, float& m, float& l, f32x16* o,
                                                bf16x2* p_new, const OperandTable<D, VTR>& tb, bool hv) {
  constexpr int DB = D / 32;
  if constexpr (SM == kSoftmaxRunningMax) {
    const float mnew = fmaxf(m, tile_row_max(s0, s1, sl2));
    const float lt = pv_with_probs<D, VTR>(vt, p_old, o, s0, s1, sl2, mnew, p_new, tb, hv);
    rescale<DB>(o, l, __builtin_amdgcn_exp2f(m - mnew));
    m = mnew;
    l += lt;
  } else if constexpr (SM == kSoftmaxFixedFirst) {
    l += pv_with_probs<D, VTR>(vt, p_old, o, s0, s1, sl2, m, p_new, tb, hv);
  } else {
    float lt = pv_with_probs<D, VTR>(vt, p_old, o, s0, s1, sl2, m, p_new, tb, hv);
    if (__ballot(!(lt <= 0x1p16f))) {  // a big jump (the first tile is not run here)
      const float mnew = fmaxf(m, ceilf(tile_row_max(s0, s1, sl2)));
      rescale<DB>(o, l, __builtin_amdgcn_exp2f(m - mnew));
      m = mnew;
      lt = tile_probs(s0, s1, sl2, m, p_new);
    }
    l += lt;
  }
}

// One workgroup (2 wavefronts x 32 query slots) per (bh, query cube); it walks
// the k selected key cubes, one cube (64 keys) per tile.  K and V^T of the
// current cubes sit in one K slot and one V slot of LDS (32 KiB per
// workgroup).  Each wavefront's tile t is: the scores S(t) = K(t) Q^T, then
// the probabilities of tile t with P(t-1) V(t-1) interleaved (the matrix pipe
// works through the softmax), so the P V of a tile runs one tile late and the
// last one after the loop.  Two barriers per tile: after the scores (K slot
// free, V(t-1) visible: the copy of K(t+1) starts and has the softmax to
// land) and after the softmax (V slot free, K(t+1) visible: the copy of V(t)
// starts and has the next scores to land).  Padded key slots of edge cubes
// are masked; output rows are scattered back to grid order, padded query
// slots are not written.  With GATED the epilogue adds gate * Oc of the
// query cube (gated merge); the last tile loads the gate rows where other
// tiles copy the next K cube.  SM selects the softmax reference policy
// (softmax_tile).  BLK is the shape of the 64-token blocks (VSA's cubes;
// sliding-tile attention's slabs).  With GRID_QK, qc and kc are the
// token-grid Q and K themselves ([BH][N][D]): the query rows are loaded by
// token (padded slots get zero rows, as in the cube-ordered copy) and the K
// tiles are copied with grid_k_copy.  With GRID_V, vct is the token-grid V
// too: its tiles are copied with grid_v_copy and the P V operands read from
// them with transpose reads (VtrSwz), so the gather need not write the
// transposed copy Vct.  The output is the same bit for bit either way.
// Cubes whose slots 32..63 are all padding (the last layer along t when
// T % 4 is 1 or 2) cost less: the second wavefront of such a query cube only
// copies and meets the barriers, and such a key cube gets the scores of its
// first 32 keys and the P V MFMAs of those keys only -- the skipped MFMAs
// would add zeros, so O and lse keep their bits.
template <int D, bool GATED, int SM = kSoftmaxGuarded, class BLK = Cube, bool GRID_QK = false, bool GRID_V = false>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) wf_vsa_fine_fwd(
    const uint16_t* __restrict__ qc, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vct, const int* __restrict__ idx, float* __restrict__ o,
    float* __restrict__ lse, const uint16_t* __restrict__ gate, const float* __restrict__ ocoarse,
    Grid3 g, int k, long plan_stride, float sl2) {
  constexpr int DB = D / 32, NPV = Pairs<D>::NPV, NQK = Pairs<D>::NQK;
  __shared__ __align__(16) char ks[Swz<D>::KB];
  __shared__ __align__(16) char vs[Swz<D>::VB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, j = lane % 32,
            half = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.C, c = item % g.C;
  const long cube_base = (long)bh * g.C;
  const int* plan = idx + bh * plan_stride + (long)c * k;  // plan_stride 0: one plan shared by all heads
  const int slot = wave * 32 + j;
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
  const long N = (long)g.T * g.H * g.W;
  const long head_row0 = (long)bh * N;
  // Edge blocks whose slots 32..63 are all padding (VSA's cubes in the last layer along t when
  // T % 4 is 1 or 2): the second wavefront of such a query block computes nothing -- it takes
  // its share of the tile copies and meets the barriers -- and such a key block costs half the
  // MFMAs.  Sliding-tile attention runs only on grids its slabs divide, so its instances leave
  // all of this out (SKIP).
  constexpr bool SKIP = BLK::BT > 1;
  const bool idle = SKIP && wave == 1 && upper_half_padded<BLK>(block_at<BLK>(g, c, (uint32_t)N));

  bf16x8 qop[D / 16];
  if (!idle) {
    if constexpr (GRID_QK) {  // a padded slot gets a zero row, as in the cube-ordered copy
      const int tq = slot_token<BLK>(g, ct, ch, cw, slot);
      const uint16_t* qr = qc + (head_row0 + (tq >= 0 ? tq : 0)) * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 u = *reinterpret_cast<const uint4*>(qr + kk * 16 + half * 8);
        qop[kk] = as_bf16x8(tq >= 0 ? u : make_uint4(0, 0, 0, 0));
      }
    } else {
      const uint16_t* qr = qc + ((cube_base + c) * 64 + slot) * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qop[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kk * 16 + half * 8));
    }
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  f32x16 s0, s1;
  bf16x2 pa[16], pb[16];  // P of the tile whose P V is pending, and of the tile being scored

  const CopyOffsets<D, 2> coff(wave, lane, 64);
  constexpr int VP = CopyOffsets<D, 2>::VPW;  // V^T copies per wavefront and tile
  const OperandTable<D, GRID_V> otab(j, half);  // every operand read's LDS offset
  // the head's cube-ordered K and V^T: every copy is range-checked against these C cubes, so a
  // plan entry outside [0, C) reads zeros (cube_copy) instead of memory beyond them
  const uint16_t* khead = GRID_QK ? kc + head_row0 * D : kc + cube_base * 64 * D;
  const uint16_t* vhead = GRID_V ? vct + head_row0 * D : vct + cube_base * D * 64;
  // the next K tile: from the cube-ordered copy, or (GRID_QK) from the token grid
  auto copy_k = [&](int cube, const BlockAt& at) __attribute__((always_inline)) {
    if constexpr (GRID_QK)
      grid_k_copy<D>(khead, (uint32_t)(N * D * 2), ks, at, g, wave, lane);
    else
      cube_copy<D, 2>(coff, khead, ks, nullptr, nullptr, cube, g.C, wave);
  };
  // the V tile of a cube: V^T from the cube-ordered copy, or (GRID_V) V from the token grid
  auto copy_v = [&](int cube, const BlockAt& at) __attribute__((always_inline)) {
    if constexpr (GRID_V)
      grid_v_copy<D>(vhead, (uint32_t)(N * D * 2), vs, at, g, wave, lane);
    else
      cube_copy<D, 2>(coff, nullptr, nullptr, vhead, vs, cube, g.C, wave);
  };
  // where the current and the next key cube lie (block_at once per cube)
  int cur = plan[0];
  BlockAt at_cur = block_at<BLK>(g, cur, (uint32_t)N), at_nxt = at_cur;
  copy_k(cur, at_cur);
  copy_v(cur, at_cur);
  wait_tile_copies_keep<VP>();  // K(0) landed; V(0) may still fly
  GatePre gp;
  // masks the padded key slots of an edge block.  Each score is rewritten through a select that
  // reads it: a plain store of -inf into an MFMA result register is a write-after-write the
  // hardware does not order against the MFMA's own late write-back, while a read waits for it.
  auto mask_keys = [&](const BlockAt& at) __attribute__((always_inline)) {
    const int lt = at.lt, lh = at.lh, lw = at.lw;
    if (lt < BLK::BT || lh < BLK::BH || lw < BLK::BW) {
      constexpr int PL = BLK::BH * BLK::BW;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = key_row(0, r, half), b = key_row(1, r, half);
        const bool ra = a / PL < lt && (a / BLK::BW) % BLK::BH < lh && a % BLK::BW < lw;
        const bool rb = b / PL < lt && (b / BLK::BW) % BLK::BH < lh && b % BLK::BW < lw;
        s0[r] = ra ? s0[r] : -INFINITY;
        s1[r] = rb ? s1[r] : -INFINITY;
      }
    }
  };
  // S = K Q^T of the current tile; with keys 32..63 all padding (upper_half_padded) only the
  // first score block is computed, the second stays zero and mask_keys sets it to -inf
  auto scores = [&](bool upper_padded) __attribute__((always_inline)) {
    if (upper_padded) mfma_run<D, NPV, NPV + NQK, 2>(vs, ks, pa, qop, oacc, s0, s1, otab);
    else mfma_run<D, NPV, NPV + NQK>(vs, ks, pa, qop, oacc, s0, s1, otab);
  };
  // tile 0: scores and probabilities (its P V runs inside tile 1's softmax)
  bool hprev = SKIP && upper_half_padded<BLK>(at_cur);  // keys 32..63 of the previous tile are padding
  barrier_nofence();                            // K(0) visible
  if (!idle) scores(hprev);                     // S = K(0) Q^T
  barrier_nofence();                            // K slot free
  if (k > 1) {
    at_nxt = block_at<BLK>(g, plan[1], (uint32_t)N);
    copy_k(plan[1], at_nxt);
  }
  if (!idle) {
    mask_keys(at_cur);
    softmax_tile<DB, SM>(s0, s1, sl2, m, l, oacc, pa);
  }
  wait_tile_copies();  // K(1) and V(0) landed
  barrier_nofence();   // K(1), V(0) visible
  // tile t >= 1.  LAST (the gated kernel's final tile, peeled off the loop so that the gate
  // registers are live only there) loads the gate rows and the coarse output for the epilogue
  // where other tiles copy the next K cube, so their latency hides behind the softmax.  EDGE
  // instances check for half-padding key blocks; the others are for runs of tiles with none,
  // in which hprev stays false.
  auto tile = [&](int t, auto last_c, auto edge_c) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_c)::value, EDGE = decltype(edge_c)::value;
    cur = plan[t];
    at_cur = at_nxt;
    const bool hcur = EDGE && SKIP && upper_half_padded<BLK>(at_cur);
    if (!idle) scores(hcur);  // S = K(t) Q^T
    wait_tile_copies();       // V(t-1) landed
    barrier_nofence();        // K slot free; V(t-1) visible
    if constexpr (LAST) {
      if (!idle)
        gate_prefetch<D, BLK>(gp, g, ct, ch, cw, wave, lane, head_row0, gate, ocoarse + (cube_base + c) * D);
    } else if (t + 1 < k) {
      at_nxt = block_at<BLK>(g, plan[t + 1], (uint32_t)N);
      copy_k(plan[t + 1], at_nxt);
    }
    if (!idle) {  // O += P(t-1) V(t-1); P(t)
      mask_keys(at_cur);
      softmax_tile_pv<D, SM, GRID_V>(vs, pa, s0, s1, sl2, m, l, oacc, pb, otab, EDGE && hprev);
    }
    wait_tile_copies();  // K(t+1) landed (or the gate rows)
    barrier_nofence();   // V slot free; K(t+1) visible
    copy_v(cur, at_cur);  // V(t)
#pragma unroll
    for (int i = 0; i < 16; ++i) pa[i] = pb[i];
    hprev = hcur;
  };
  // A plan in ascending order (as wf_vsa_topk writes it) lists the last layer's cubes, the
  // half-padding ones, last: the tiles before the first of them run without the checks.
  const int tend = GATED ? k - 1 : k;
  int t = 1;
  for (; t < tend && !hprev && !(SKIP && upper_half_padded<BLK>(at_nxt)); ++t)
    tile(t, std::false_type(), std::false_type());
  for (; t < tend; ++t) tile(t, std::false_type(), std::true_type());
  if constexpr (GATED) {
    if (k > 1) tile(k - 1, std::true_type(), std::true_type());
  }
  wait_tile_copies();  // V(k-1) landed
  barrier_nofence();   // V(k-1) visible
  if constexpr (GATED) {  // a single tile had no later tile to load them in
    if (k == 1 && !idle)
      gate_prefetch<D, BLK>(gp, g, ct, ch, cw, wave, lane, head_row0, gate, ocoarse + (cube_base + c) * D);
  }
  if (!idle) {  // O += P(k-1) V(k-1)
    if (hprev) mfma_run<D, 0, NPV / 2>(vs, ks, pa, qop, oacc, s0, s1, otab);
    else mfma_run<D, 0, NPV>(vs, ks, pa, qop, oacc, s0, s1, otab);
  }
  wait_tile_copies();  // the gate rows (k = 1)
  barrier_nofence();   // every wavefront is done with both slots
  if (idle) return;    // no query row to write
  const float lt = l + __shfl_xor(l, 32);
  fine_epilogue<D, GATED, BLK>(oacc, 1.f / lt, wave == 0 ? ks : vs, j, half, g, ct, ch, cw, wave, head_row0, o, gp);
  const int tok = slot_token<BLK>(g, ct, ch, cw, slot);
  if (lse && tok >= 0 && half == 0) lse[head_row0 + tok] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
}

// ---------------------------------------------------------------- sliding-tile plan
// Sliding-tile attention ("推理优化", WorldFoundry docs, approximate attention,
// entry "sta": weight-free, accepted only on its tuned grids; tile and window
// sizes are not given there).  Tiles are 6x8x8 tokens, which both accepted
// grids divide exactly; a query tile attends to the tiles of a (wt, wh, ww)
// window that starts on each axis at clamp(c - (w-1)/2, 0, n - w) -- centred
// where it fits, pushed inward at the edges.  The fine stage works on 1x8x8
// slabs (64 tokens), six to a tile along t, so slab (st, sh, sw) of tile
// (st/6, sh, sw) takes the 6*wt*wh*ww slabs of that tile's window, listed in
// ascending order.  Threads [0, C*ks) write that slab plan (C slabs, ks
// entries each); with tile_plan, threads past it write the tile-level plan
// [tiles][wt*wh*ww] (tile id (tt*nh + th)*nw + tw) for the caller.
__global__ void __launch_bounds__(256) wf_sta_plan(int* __restrict__ slab_plan, int* __restrict__ tile_plan,
                                                   Grid3 g, int wt, int wh, int ww) {
  constexpr int TT = 6;  // slabs per tile along t
  const int kt = wt * wh * ww, ks = TT * kt, ntt = g.nt / TT;
  const long id = (long)blockIdx.x * 256 + threadIdx.x, nslab = (long)g.C * ks;
  if (id < nslab) {
    const int c = (int)(id / ks), e = (int)(id % ks);
    int st, sh, sw;
    cube_coords(g, c, st, sh, sw);
    const int t0 = min(max(st / TT - (wt - 1) / 2, 0), ntt - wt);
    const int h0 = min(max(sh - (wh - 1) / 2, 0), g.nh - wh);
    const int w0 = min(max(sw - (ww - 1) / 2, 0), g.nw - ww);
    const int iw = e % ww, ih = (e / ww) % wh, js = e / (ww * wh);  // js = it * TT + slab within the tile
    slab_plan[id] = ((t0 * TT + js) * g.nh + (h0 + ih)) * g.nw + (w0 + iw);
  } else if (tile_plan && id < nslab + (long)ntt * g.nh * g.nw * kt) {
    const long r = id - nslab;
    const int c = (int)(r / kt), j = (int)(r % kt);
    const int tw = c % g.nw, th = (c / g.nw) % g.nh, tt = c / (g.nw * g.nh);
    const int t0 = min(max(tt - (wt - 1) / 2, 0), ntt - wt);
    const int h0 = min(max(th - (wh - 1) / 2, 0), g.nh - wh);
    const int w0 = min(max(tw - (ww - 1) / 2, 0), g.nw - ww);
    const int jt = j / (wh * ww), jh = (j / ww) % wh, jw = j % ww;
    tile_plan[r] = ((t0 + jt) * g.nh + (h0 + jh)) * g.nw + (w0 + jw);
  }
}

// ---------------------------------------------------------------- plan check
__global__ void wf_vsa_flag_clear(int* flag) { *flag = 0; }

__global__ void __launch_bounds__(256) wf_vsa_check_plan(const int* __restrict__ idx, long rows,
                                                         int C, int k, int* flag) {
  const long row = (long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int* p = idx + row * k;
  int prev = -1;
  bool bad = false;
  for (int i = 0; i < k; ++i) {
    const int x = p[i];
    bad |= (x <= prev) || (x >= C);
    prev = x;
  }
  if (bad) atomicOr(flag, 1);
}

// ---------------------------------------------------------------- host side
VsaLayout vsa_layout(int BH, int T, int H, int W, int D) {
  const Grid3 g = make_grid<Cube>(T, H, W);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  VsaLayout L{};
  L.C = g.C;
  const size_t tok = (size_t)BH * g.C * 64 * D * 2;
  L.qc = 0;
  L.kc = L.qc + up(tok);
  L.vct = L.kc + up(tok);
  L.qbar = L.vct + up(tok);
  L.kbar = L.qbar + up((size_t)BH * mean_blocks(g.C) * 32 * D * 3 * 2);
  L.vbt = L.kbar + up((size_t)BH * mean_blocks(g.C) * 32 * D * 3 * 2);
  L.scores = L.vbt + up((size_t)2 * BH * D * g.Cs * 2);
  L.stat = L.scores + up((size_t)BH * g.C * g.Cs * 4);
  L.ocoarse = L.stat + up((size_t)BH * g.C * 8);
  L.flag = L.ocoarse + up((size_t)BH * g.C * D * 4);
  L.total = L.flag + 256;
  return L;
}

// Coarse scores and per-row top-k of every head (wf_vsa_scores, then wf_vsa_topk), from the
// cube means in the workspace.
static hipError_t launch_scores_topk(const uint16_t* qbar, const uint16_t* kbar, float* sc, float* scores_out, int* idx,
                                     float2* stat, int BH, const Grid3& g, float scale, int topk, hipStream_t s) {
  const int ntr = (g.C + 127) / 128, ntc = (g.Cs + 127) / 128;
  hipError_t e = wf_launch("wf_vsa_scores", s, [&] {
    hipLaunchKernelGGL(wf_vsa_scores<128>, dim3((unsigned)((long)BH * ntr * ntc)), dim3(256), 0, s, qbar,
                       kbar, sc, scores_out, g.C, g.Cs, ntr, ntc, scale);
  });
  if (e != hipSuccess) return e;
  const long rows = (long)BH * g.C;
  const dim3 grid((unsigned)((rows + 3) / 4));
  // E candidates per lane: the smallest instantiated E with 64 * E >= C (the bitwise search costs
  // E ballots per bit, so padding E wastes work)
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, sc, idx, stat, rows, g.C, g.Cs, topk);
  };
  return wf_launch("wf_vsa_topk", s, [&] {
    const int e = (g.C + 63) / 64;
    if (e <= 2) go(wf_vsa_topk<2>);
    else if (e <= 4) go(wf_vsa_topk<4>);
    else if (e <= 8) go(wf_vsa_topk<8>);
    else if (e <= 10) go(wf_vsa_topk<10>);
    else if (e <= 12) go(wf_vsa_topk<12>);
    else if (e <= 16) go(wf_vsa_topk<16>);
    else if (e <= 20) go(wf_vsa_topk<20>);
    else if (e <= 24) go(wf_vsa_topk<24>);
    else if (e <= 32) go(wf_vsa_topk<32>);
    else if (e <= 48) go(wf_vsa_topk<48>);
    else go(wf_vsa_topk<64>);
  });
}

hipError_t launch_vsa_coarse(const void* q, const void* k, const void* v, int BH, int T, int H,
                             int W, int D, float scale, int topk, double rope_theta,
                             int rope_precision, int* idx, float* scores_out, void* ws, hipStream_t s) {
  const Grid3 g = make_grid<Cube>(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  auto qc = reinterpret_cast<uint16_t*>(w + L.qc), kc = reinterpret_cast<uint16_t*>(w + L.kc),
       vct = reinterpret_cast<uint16_t*>(w + L.vct);
  auto qbar = reinterpret_cast<uint16_t*>(w + L.qbar), kbar = reinterpret_cast<uint16_t*>(w + L.kbar);
  auto vbt = reinterpret_cast<uint16_t*>(w + L.vbt);
  auto sc = reinterpret_cast<float*>(w + L.scores);
  auto stat = reinterpret_cast<float2*>(w + L.stat);
  auto gather = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * g.C)), dim3(256), 0, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), qc, kc, vct, qbar,
                       kbar, vbt, g, rope_theta);
  };
  hipError_t e;
  if (rope_theta > 0.0 && rope_precision == 64)
    e = wf_launch("wf_vsa_gather_rope_fp64", s, [&] { gather(wf_vsa_gather<128, 64>); });
  else if (rope_theta > 0.0)
    e = wf_launch("wf_vsa_gather_rope", s, [&] { gather(wf_vsa_gather<128, 32>); });
  else
    e = wf_launch("wf_vsa_gather", s, [&] { gather(wf_vsa_gather<128, 0>); });
  if (e != hipSuccess) return e;
  return launch_scores_topk(qbar, kbar, sc, scores_out, idx, stat, BH, g, scale, topk, s);
}

hipError_t launch_vsa_check(const int* idx, int BH, int C, int topk, void* ws, size_t flag_off,
                            hipStream_t s, int* bad) {
  int* flag = reinterpret_cast<int*>(static_cast<char*>(ws) + flag_off);
  hipLaunchKernelGGL(wf_vsa_flag_clear, dim3(1), dim3(1), 0, s, flag);
  const long rows = (long)BH * C;
  hipLaunchKernelGGL(wf_vsa_check_plan, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, idx,
                     rows, C, topk, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int h = 0;
  e = hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  *bad = h;
  return e;
}

hipError_t launch_vsa_fine(const void* ws, const int* idx, int BH, int T, int H, int W, int D,
                           float scale, int topk, int softmax_mode, float* o, float* lse, hipStream_t s) {
  const Grid3 g = make_grid<Cube>(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  const char* w = static_cast<const char*>(ws);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * g.C)), dim3(128), 0, s,
                       reinterpret_cast<const uint16_t*>(w + L.qc), reinterpret_cast<const uint16_t*>(w + L.kc),
                       reinterpret_cast<const uint16_t*>(w + L.vct), idx, o, lse, nullptr, nullptr, g, topk,
                       (long)g.C * topk, scale * kLog2e);
  };
  if (softmax_mode == kSoftmaxRunningMax)
    return wf_launch("wf_vsa_fine_running_max", s, [&] { go(wf_vsa_fine_fwd<128, false, kSoftmaxRunningMax>); });
  if (softmax_mode == kSoftmaxFixedFirst)
    return wf_launch("wf_vsa_fine_fixed_first", s, [&] { go(wf_vsa_fine_fwd<128, false, kSoftmaxFixedFirst>); });
  return wf_launch("wf_vsa_fine", s, [&] { go(wf_vsa_fine_fwd<128, false, kSoftmaxGuarded>); });
}

// The coarse-branch output O_c of every head from the workspace's scores, row statistics and
// operand-ordered cube means of V.
static hipError_t launch_coarse_out(const char* w, const VsaLayout& L, const Grid3& g, int BH, float* oc,
                                    hipStream_t s) {
  const int rblocks = (g.C + 31) / 32;
  return wf_launch("wf_vsa_coarse_out", s, [&] {
    hipLaunchKernelGGL(wf_vsa_coarse_out<128>, dim3((unsigned)(BH * rblocks)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(w + L.scores),
                       reinterpret_cast<const float2*>(w + L.stat),
                       reinterpret_cast<const uint16_t*>(w + L.vbt), oc, g.C, g.Cs, rblocks);
  });
}

// VSA in one call: the gather writes only the cube means (no cube-ordered Q, K or V), the coarse
// scores and top-k fill idx, and the fine stage reads Q, K and V from the token grid; with a gate,
// the coarse-branch output and the gated merge as in launch_vsa_fine_gated.
hipError_t launch_vsa_onecall(const void* q, const void* k, const void* v, int BH, int T, int H, int W, int D,
                              float scale, int topk, int* idx, const void* gate, float* o, float* lse,
                              float* o_coarse, void* ws, hipStream_t s) {
  const Grid3 g = make_grid<Cube>(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  auto qbar = reinterpret_cast<uint16_t*>(w + L.qbar), kbar = reinterpret_cast<uint16_t*>(w + L.kbar);
  auto vbt = reinterpret_cast<uint16_t*>(w + L.vbt);
  auto qg = static_cast<const uint16_t*>(q), kg = static_cast<const uint16_t*>(k),
       vg = static_cast<const uint16_t*>(v);
  // the means only, and the mean of V for the coarse branch when there is a gate
  auto gather = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * g.C)), dim3(256), 0, s, qg, kg, vg, nullptr, nullptr, nullptr,
                       qbar, kbar, vbt, g, 0.0);
  };
  hipError_t e = wf_launch("wf_vsa_gather", s, [&] {
    if (gate) gather(wf_vsa_gather<128, 0, Cube, true, kOutVbar>);
    else gather(wf_vsa_gather<128, 0, Cube, true, 0>);
  });
  if (e != hipSuccess) return e;
  e = launch_scores_topk(qbar, kbar, reinterpret_cast<float*>(w + L.scores), nullptr, idx,
                         reinterpret_cast<float2*>(w + L.stat), BH, g, scale, topk, s);
  if (e != hipSuccess) return e;
  auto fine = [&](auto kernel, const uint16_t* gt, const float* oc) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * g.C)), dim3(128), 0, s, qg, kg, vg, idx, o, lse, gt, oc, g, topk,
                       (long)g.C * topk, scale * kLog2e);
  };
  if (!gate)
    return wf_launch("wf_vsa_fine", s, [&] {
      fine(wf_vsa_fine_fwd<128, false, kSoftmaxGuarded, Cube, true, true>, nullptr, nullptr);
    });
  float* oc = o_coarse ? o_coarse : reinterpret_cast<float*>(w + L.ocoarse);
  e = launch_coarse_out(w, L, g, BH, oc, s);
  if (e != hipSuccess) return e;
  return wf_launch("wf_vsa_fine_gated", s, [&] {
    fine(wf_vsa_fine_fwd<128, true, kSoftmaxGuarded, Cube, true, true>, static_cast<const uint16_t*>(gate), oc);
  });
}

// Sliding-tile attention workspace: the slab-ordered Q, K and V^T, then the slab plan shared by
// all heads.  k is the window's tile count wt*wh*ww.
StaLayout sta_layout(int BH, int T, int H, int W, int D, int k) {
  const Grid3 g = make_grid<Slab>(T, H, W);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  StaLayout L{};
  const size_t tok = (size_t)BH * g.C * 64 * D * 2;
  L.qc = 0;
  L.kc = L.qc + up(tok);
  L.vct = L.kc + up(tok);
  L.plan = L.vct + up(tok);
  L.total = L.plan + up((size_t)g.C * 6 * k * 4);
  return L;
}

int sta_slabs(int T, int H, int W) { return make_grid<Slab>(T, H, W).C; }

hipError_t launch_sta(const void* q, const void* k, const void* v, int BH, int T, int H, int W, int D,
                      float scale, int wt, int wh, int ww, float* o, float* lse, int* plan_out, void* ws,
                      hipStream_t s) {
  const Grid3 g = make_grid<Slab>(T, H, W);
  const int kt = wt * wh * ww, ks = 6 * kt;
  const StaLayout L = sta_layout(BH, T, H, W, D, kt);
  char* w = static_cast<char*>(ws);
  auto qc = reinterpret_cast<uint16_t*>(w + L.qc), kc = reinterpret_cast<uint16_t*>(w + L.kc),
       vct = reinterpret_cast<uint16_t*>(w + L.vct);
  int* plan = reinterpret_cast<int*>(w + L.plan);
  hipError_t e = wf_launch("wf_sta_gather", s, [&] {
    hipLaunchKernelGGL((wf_vsa_gather<128, 0, Slab, false>), dim3((unsigned)(BH * g.C)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), qc, kc, vct, nullptr, nullptr, nullptr, g, 0.0);
  });
  if (e != hipSuccess) return e;
  const long threads = (long)g.C * ks + (plan_out ? (long)(g.C / 6) * kt : 0);
  e = wf_launch("wf_sta_plan", s, [&] {
    hipLaunchKernelGGL(wf_sta_plan, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, plan, plan_out, g,
                       wt, wh, ww);
  });
  if (e != hipSuccess) return e;
  return wf_launch("wf_sta_fine", s, [&] {
    hipLaunchKernelGGL((wf_vsa_fine_fwd<128, false, kSoftmaxGuarded, Slab>), dim3((unsigned)(BH * g.C)), dim3(128),
                       0, s, qc, kc, vct, plan, o, lse, nullptr, nullptr, g, ks, 0L, scale * kLog2e);
  });
}

hipError_t launch_vsa_fine_gated(void* ws, const int* idx, const void* gate, int BH, int T, int H,
                                 int W, int D, float scale, int topk, float* o, float* lse,
                                 float* o_coarse, hipStream_t s) {
  const Grid3 g = make_grid<Cube>(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  float* oc = o_coarse ? o_coarse : reinterpret_cast<float*>(w + L.ocoarse);
  hipError_t e = launch_coarse_out(w, L, g, BH, oc, s);
  if (e != hipSuccess) return e;
  return wf_launch("wf_vsa_fine_gated", s, [&] {
    hipLaunchKernelGGL((wf_vsa_fine_fwd<128, true>), dim3((unsigned)(BH * g.C)), dim3(128), 0, s,
                       reinterpret_cast<const uint16_t*>(w + L.qc),
                       reinterpret_cast<const uint16_t*>(w + L.kc),
                       reinterpret_cast<const uint16_t*>(w + L.vct), idx, o, lse,
                       static_cast<const uint16_t*>(gate), oc, g, topk, (long)g.C * topk, scale * kLog2e);
  });
}

}  // namespace wf
