// Video Sparse Attention (VSA) on gfx950: cube gather and pooling, coarse
// cube scores, per-cube top-k and fine block-sparse attention.
//
// Operation: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "VSA
// selects cubes": pad the T x H x W grid to multiples of 4, cut it into 4x4x4
// cubes of 64 tokens, score cube-mean queries against cube-mean keys, keep the
// top-k key cubes of every query cube, then run token-level attention of each
// query cube over those cubes only.  Section "Roofline analysis set the 3.35
// ms target" counts one output tile per (query cube, head).
#include "wf_attn.h"
#include "wf_device.hpp"
#include "wf_launch.hpp"
#include "wf_rope.hpp"

namespace wf {

static_assert(kSoftmaxGuarded == WF_SOFTMAX_GUARDED && kSoftmaxRunningMax == WF_SOFTMAX_RUNNING_MAX &&
                  kSoftmaxFixedFirst == WF_SOFTMAX_FIXED_FIRST_TILE,
              "softmax policy numbers of the C ABI and the kernels");

// Cs: the cube count rounded up to a multiple of 32, the row stride of the
// coarse scores and of the transposed cube means of V in the workspace.
struct Grid3 {
  int T, H, W, nt, nh, nw, C, Cs;
};

static Grid3 make_grid(int T, int H, int W) {
  Grid3 g{T, H, W, (T + 3) / 4, (H + 3) / 4, (W + 3) / 4, 0, 0};
  g.C = g.nt * g.nh * g.nw;
  g.Cs = (g.C + 31) / 32 * 32;
  return g;
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Element offset of (part, head, key cube, head dim) in the cube means of V,
// stored in the lane order of the coarse-branch MFMA's A operand so that one
// load of a wavefront reads 1 KiB contiguously: [part hi/lo][bh][key step of
// 16][dim block of 32][lane 0..63][8 key cubes], lane = dim % 32 + 32 * (key % 16 / 8).
__device__ __forceinline__ long vbar_index(int part, int bh, int BH, int Cs, int key, int d) {
  const int lane = d % 32 + 32 * ((key % 16) / 8);
  return ((((long)part * BH + bh) * (Cs / 16) + key / 16) * 4 + d / 32) * 512 + lane * 8 + key % 8;
}

// Token of slot s in cube (ct, ch, cw), or -1 for a padded slot.
__device__ __forceinline__ int slot_token(const Grid3& g, int ct, int ch, int cw, int s) {
  const int t = ct * 4 + (s >> 4), h = ch * 4 + ((s >> 2) & 3), w = cw * 4 + (s & 3);
  return (t < g.T && h < g.H && w < g.W) ? (t * g.H + h) * g.W + w : -1;
}

__device__ __forceinline__ void cube_coords(const Grid3& g, int c, int& ct, int& ch, int& cw) {
  cw = c % g.nw;
  ch = (c / g.nw) % g.nh;
  ct = c / (g.nw * g.nh);
}

// ---------------------------------------------------------------- gather + pool
// One workgroup per (bh, cube).  Writes Qc, Kc [BH][C][64][D] (padded slots
// zero), Vct [BH][C][D][64] (slots in perm16 order), the fp32 means of Q and K
// over the cube's real tokens, and the fp32 mean of V split into two bf16
// parts, hi = bf16(mean) and lo = bf16(mean - hi), at key cube c of the
// operand-ordered means (vbar_index; key cubes C..Cs-1 are zeroed, so the
// coarse-branch product may run over whole 32-wide steps).  With ROPE, Q and
// K are rotated by the 3D RoPE (wf_rope.hpp) on the way in, so everything
// downstream (cube means, scores, the fine stage) sees the rotated vectors;
// the cube's 4 t, 4 h and 4 w coordinates need one table of 4*(t2+h2+w2)
// (cos, sin) pairs, one fp64 sincos per thread.  ROPE is the rotation's
// precision (32 or 64), 0 for none.
template <int D, int ROPE>
__global__ void __launch_bounds__(256) wf_vsa_gather(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qc, uint16_t* __restrict__ kc, uint16_t* __restrict__ vct,
    float* __restrict__ qbar, float* __restrict__ kbar, uint16_t* __restrict__ vbt, Grid3 g,
    double theta) {
  constexpr int ROWCH = D / 8;            // 16-byte chunks per row
  constexpr int RSTEP = 256 / ROWCH;      // rows covered by one pass of the workgroup
  constexpr int VSTR = D + 2;
  constexpr RopeSplit sp = rope_split(D);
  constexpr int NTAB = ROPE ? 4 * (sp.t2 + sp.h2 + sp.w2) : 1;
  using CS = RopeCS<ROPE == 64 ? 64 : 32>;
  __shared__ float red[RSTEP][D];
  __shared__ uint16_t vtile[64 * VSTR];
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
  const int count = min(4, g.T - 4 * ct) * min(4, g.H - 4 * ch) * min(4, g.W - 4 * cw);

  for (int which = 0; which < 3; ++which) {
    const uint16_t* src = (which == 0 ? q : which == 1 ? k : v) + (long)bh * N * D;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 64 / RSTEP; ++i) {
      const int s = r0 + i * RSTEP;
      const int tok = slot_token(g, ct, ch, cw, s);
      uint4 u = make_uint4(0, 0, 0, 0);
      if (tok >= 0) u = *reinterpret_cast<const uint4*>(src + (long)tok * D + c16 * 8);
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
        uint16_t* dst = (which == 0 ? qc : kc) + (cube_row0 + s) * D + c16 * 8;
        *reinterpret_cast<uint4*>(dst) = u;
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) vtile[s * VSTR + c16 * 8 + t] = e[t];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += __uint_as_float((uint32_t)e[t] << 16);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) red[r0][c16 * 8 + t] = acc[t];
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < RSTEP; ++r) sum += red[r][tid];
      const float mean = sum / (float)count;
      if (which < 2) {
        (which == 0 ? qbar : kbar)[((long)bh * g.C + c) * D + tid] = mean;
      } else {
        static_assert(D == 128, "four 32-wide head-dim blocks");
        const int BH = gridDim.x / g.C;  // gridDim.x = BH * C
        const __bf16 h16 = (__bf16)mean;
        vbt[vbar_index(0, bh, BH, g.Cs, c, tid)] = __builtin_bit_cast(uint16_t, h16);
        vbt[vbar_index(1, bh, BH, g.Cs, c, tid)] = __builtin_bit_cast(uint16_t, (__bf16)(mean - (float)h16));
        for (int x = g.C + c; x < g.Cs; x += g.C)
          vbt[vbar_index(0, bh, BH, g.Cs, x, tid)] = vbt[vbar_index(1, bh, BH, g.Cs, x, tid)] = 0;
      }
    }
    __syncthreads();
    if (which == 2) {
      uint16_t* dst = vct + ((long)bh * g.C + c) * D * 64;
      for (int id = tid; id < D * 8; id += 256) {
        const int d = id / 8, pc = id % 8;
        uint16_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = vtile[perm16(pc * 8 + t) * VSTR + d];
        *reinterpret_cast<uint4*>(dst + d * 64 + pc * 8) = *reinterpret_cast<const uint4*>(e);
      }
    }
  }
}

// ---------------------------------------------------------------- coarse scores
// S[bh][c][c'] = scale * sum_d Qbar[c][d] Kbar[c'][d] in fp32 on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32).  One workgroup (4 wavefronts) per 128x128
// tile of S, a 64x64 tile (2x2 blocks of 32x32) per wavefront, so each operand
// row a wavefront loads feeds two blocks.  The sum over d is order-free, so
// lane half h takes d = 32u + 16h + s at step s of chunk u for both operands:
// each lane's operands are 16 consecutive floats of one row, read straight
// from memory (L2) as four 16-byte loads, no LDS.  s has row stride Cs and -inf in
// columns C..Cs-1; s_user (optional) gets the same scores with row stride C.
template <int D>
__global__ void __launch_bounds__(256) wf_vsa_scores(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar,
                                                     float* __restrict__ s, float* __restrict__ s_user,
                                                     int C, int Cs, int ntr, int ntc, float scale) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, j = lane % 32,
            h = lane / 32;
  const int per_head = ntr * ntc;
  const int bh = blockIdx.x / per_head, rem = blockIdx.x % per_head;
  // workgroup tile 128 x 128, wavefront tile 64 x 64 = 2 x 2 blocks of 32 x 32
  const int r0 = (rem / ntc) * 128 + (wave >> 1) * 64, c0 = (rem % ntc) * 128 + (wave & 1) * 64;
  const float* arow[2];
  const float* brow[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    arow[x] = qbar + ((long)bh * C + min(r0 + 32 * x + j, C - 1)) * D + h * 16;
    brow[x] = kbar + ((long)bh * C + min(c0 + 32 * x + j, C - 1)) * D + h * 16;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.f;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    f32x4 a[2][4], bq[2][4];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        a[x][v] = *reinterpret_cast<const f32x4*>(arow[x] + u * 32 + v * 4);
        bq[x][v] = *reinterpret_cast<const f32x4*>(brow[x] + u * 32 + v * 4);
      }
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x][st / 4][st % 4], bq[y][st / 4][st % 4], acc[x][y], 0, 0, 0);
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
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
    if (cnt >= k) thr = cand;
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

// Fine-stage epilogue: the normalised output rows of a wavefront go through
// its own LDS slot (32 rows x D fp32 = 16 KiB, the K or V slot, free once the
// sweep is done), so that global stores cover two whole token rows per
// instruction instead of 16 bytes of 32 different rows.  In LDS, row r's
// 16-byte chunk c sits at chunk c ^ (r % 32), which keeps both the scattered
// writes and the row reads free of bank conflicts.  With GATED the merge
// O = O_fine + gate * Oc is applied on the way out, where the gate is read
// row-contiguously as well.
template <int D, bool GATED>
__device__ __forceinline__ void fine_epilogue(const f32x16* o, float inv, char* slot_lds, int j, int half,
                                              const Grid3& g, int ct, int ch, int cw, int wave, long head_row0,
                                              float* __restrict__ out, const uint16_t* __restrict__ gate,
                                              const float* __restrict__ ocube) {
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
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + lane / 32;  // row inside this wavefront's 32
    const int tok = slot_token(g, ct, ch, cw, wave * 32 + r);
    float4 v = *reinterpret_cast<const float4*>(lds + r * D + ((c ^ r) * 4));
    if (tok >= 0) {
      const long row = head_row0 + tok;
      if constexpr (GATED) {
        const float4 c4 = *reinterpret_cast<const float4*>(ocube + c * 4);
        const uint2 g2 = *reinterpret_cast<const uint2*>(gate + row * D + c * 4);
        v.x = __builtin_fmaf(__uint_as_float(g2.x << 16), c4.x, v.x);
        v.y = __builtin_fmaf(__uint_as_float(g2.x & 0xFFFF0000u), c4.y, v.y);
        v.z = __builtin_fmaf(__uint_as_float(g2.y << 16), c4.z, v.z);
        v.w = __builtin_fmaf(__uint_as_float(g2.y & 0xFFFF0000u), c4.w, v.w);
      }
      *reinterpret_cast<float4*>(out + row * D + c * 4) = v;
    }
  }
}

// ---------------------------------------------------------------- fine stage
// One workgroup (2 wavefronts x 32 query slots) per (bh, query cube); it walks
// the k selected key cubes, one cube (64 keys) per tile.  K and V^T of the
// current cube sit in one K slot and one V slot of LDS (32 KiB, so several
// workgroups share a CU and hide each other's latency).  The slots have
// separate lifetimes: the copy of the next K cube starts as soon as both
// wavefronts have their scores and is waited for at the next tile's start; the
// copy of the next V cube starts once both have accumulated P V and is waited
// for only before the next P V, so it lands behind the next tile's scores and
// softmax.  Padded key slots of edge cubes are masked; output rows are
// scattered back to grid order, padded query slots are not written.  With
// GATED the epilogue adds gate * Oc of the query cube (gated merge).  SM
// selects the softmax reference policy (softmax_tile).
template <int D, bool GATED, int SM = kSoftmaxGuarded>
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

  bf16x8 qop[D / 16];
  {
    const uint16_t* qr = qc + ((cube_base + c) * 64 + slot) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qop[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + kk * 16 + half * 8));
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  f32x16 s0, s1;
  bf16x2 p2[16];

  int cur = plan[0];
  const CopyOffsets<D, 2> coff(wave, lane, 64);
  constexpr uint32_t CUBE_BYTES = 64u * D * 2;
  constexpr int KP = CopyOffsets<D, 2>::KPW, VP = CopyOffsets<D, 2>::VPW;  // copies per wavefront and tile
  tile_copy<D, 2>(coff, kc + (cube_base + cur) * 64 * D, 64, ks, nullptr, 0, 0, nullptr, wave);
  tile_copy<D, 2>(coff, nullptr, 0, nullptr, vct + (cube_base + cur) * D * 64, 64, CUBE_BYTES, vs, wave);
  wait_tile_copies_keep<VP>();  // K(0) landed; V(0) may still fly
  for (int t = 0; t < k; ++t) {
    barrier_nofence();  // K(t) visible
    mfma_run<D, NPV, NPV + NQK>(vs, ks, p2, qop, oacc, s0, s1, j, half);  // S = K(t) Q^T
    barrier_nofence();                                                     // K slot free
    const int nxt = t + 1 < k ? plan[t + 1] : cur;  // past the end: a harmless copy of the last cube
    tile_copy<D, 2>(coff, kc + (cube_base + nxt) * 64 * D, 64, ks, nullptr, 0, 0, nullptr, wave);
    int kt, kh, kw;
    cube_coords(g, cur, kt, kh, kw);
    const int lt = g.T - 4 * kt, lh = g.H - 4 * kh, lw = g.W - 4 * kw;
    if (lt < 4 || lh < 4 || lw < 4) {  // edge cube: mask padded key slots
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = key_row(0, r, half), b = key_row(1, r, half);
        if (!((a >> 4) < lt && ((a >> 2) & 3) < lh && (a & 3) < lw)) s0[r] = -INFINITY;
        if (!((b >> 4) < lt && ((b >> 2) & 3) < lh && (b & 3) < lw)) s1[r] = -INFINITY;
      }
    }
    softmax_tile<DB, SM>(s0, s1, sl2, m, l, oacc, p2);
    wait_tile_copies_keep<KP>();  // V(t) landed (it had the scores and the softmax to do so); K(t+1) may fly
    barrier_nofence();            // V(t) visible
    mfma_run<D, 0, NPV>(vs, ks, p2, qop, oacc, s0, s1, j, half);  // O += P V(t)
    barrier_nofence();                                             // V slot free
    tile_copy<D, 2>(coff, nullptr, 0, nullptr, vct + (cube_base + nxt) * D * 64, 64, CUBE_BYTES, vs, wave);
    wait_tile_copies_keep<VP>();  // K(t+1) landed; V(t+1) may fly
    cur = nxt;
  }
  wait_tile_copies();  // this wavefront's copies (the last ones are redundant) have landed
  barrier_nofence();   // every wavefront is done with both slots
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
  const long head_row0 = (long)bh * g.T * g.H * g.W;
  const float lt = l + __shfl_xor(l, 32);
  fine_epilogue<D, GATED>(oacc, 1.f / lt, wave == 0 ? ks : vs, j, half, g, ct, ch, cw, wave, head_row0, o,
                          gate, GATED ? ocoarse + (cube_base + c) * D : nullptr);
  const int tok = slot_token(g, ct, ch, cw, slot);
  if (lse && tok >= 0 && half == 0) lse[head_row0 + tok] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
}

// ---------------------------------------------------------------- sliding-tile plan
// Sliding-tile attention ("推理优化", WorldFoundry docs, approximate attention,
// entry "sta": weight-free, on tuned grids; tile and window sizes are not
// given there): query cube c attends to the cubes of a (wt, wh, ww)-cube
// window, on each axis starting at clamp(c - (w-1)/2, 0, n - w) -- centred
// where it fits, pushed inward at the edges -- so every row has wt*wh*ww
// cubes.  One thread per (cube, slot); slots run row-major over the window,
// which lists the cubes in ascending order.
__global__ void __launch_bounds__(256) wf_sta_plan(int* __restrict__ plan, Grid3 g, int wt, int wh, int ww) {
  const int k = wt * wh * ww;
  const long id = (long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long)g.C * k) return;
  const int c = (int)(id / k), j = (int)(id % k);
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
  const int t0 = min(max(ct - (wt - 1) / 2, 0), g.nt - wt);
  const int h0 = min(max(ch - (wh - 1) / 2, 0), g.nh - wh);
  const int w0 = min(max(cw - (ww - 1) / 2, 0), g.nw - ww);
  const int jt = j / (wh * ww), jh = (j / ww) % wh, jw = j % ww;
  plan[id] = ((t0 + jt) * g.nh + (h0 + jh)) * g.nw + (w0 + jw);
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
  const Grid3 g = make_grid(T, H, W);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  VsaLayout L{};
  L.C = g.C;
  const size_t tok = (size_t)BH * g.C * 64 * D * 2;
  L.qc = 0;
  L.kc = L.qc + up(tok);
  L.vct = L.kc + up(tok);
  L.qbar = L.vct + up(tok);
  L.kbar = L.qbar + up((size_t)BH * g.C * D * 4);
  L.vbt = L.kbar + up((size_t)BH * g.C * D * 4);
  L.scores = L.vbt + up((size_t)2 * BH * D * g.Cs * 2);
  L.stat = L.scores + up((size_t)BH * g.C * g.Cs * 4);
  L.ocoarse = L.stat + up((size_t)BH * g.C * 8);
  L.flag = L.ocoarse + up((size_t)BH * g.C * D * 4);
  L.total = L.flag + 256;
  return L;
}

hipError_t launch_vsa_coarse(const void* q, const void* k, const void* v, int BH, int T, int H,
                             int W, int D, float scale, int topk, double rope_theta,
                             int rope_precision, int* idx, float* scores_out, void* ws, hipStream_t s) {
  const Grid3 g = make_grid(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  auto qc = reinterpret_cast<uint16_t*>(w + L.qc), kc = reinterpret_cast<uint16_t*>(w + L.kc),
       vct = reinterpret_cast<uint16_t*>(w + L.vct);
  auto qbar = reinterpret_cast<float*>(w + L.qbar), kbar = reinterpret_cast<float*>(w + L.kbar);
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
  const int ntr = (g.C + 127) / 128, ntc = (g.Cs + 127) / 128;
  e = wf_launch("wf_vsa_scores", s, [&] {
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
  const Grid3 g = make_grid(T, H, W);
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

// Sliding-tile attention workspace: the gather's regions, then the shared plan.
StaLayout sta_layout(int BH, int T, int H, int W, int D, int k) {
  const Grid3 g = make_grid(T, H, W);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  StaLayout L{};
  const size_t tok = (size_t)BH * g.C * 64 * D * 2;
  L.qc = 0;
  L.kc = L.qc + up(tok);
  L.vct = L.kc + up(tok);
  L.qbar = L.vct + up(tok);
  L.kbar = L.qbar + up((size_t)BH * g.C * D * 4);
  L.vbt = L.kbar + up((size_t)BH * g.C * D * 4);
  L.plan = L.vbt + up((size_t)2 * BH * D * g.Cs * 2);
  L.total = L.plan + up((size_t)g.C * k * 4);
  return L;
}

hipError_t launch_sta(const void* q, const void* k, const void* v, int BH, int T, int H, int W, int D,
                      float scale, int wt, int wh, int ww, float* o, float* lse, int* plan_out, void* ws,
                      hipStream_t s) {
  const Grid3 g = make_grid(T, H, W);
  const int kk = wt * wh * ww;
  const StaLayout L = sta_layout(BH, T, H, W, D, kk);
  char* w = static_cast<char*>(ws);
  auto qc = reinterpret_cast<uint16_t*>(w + L.qc), kc = reinterpret_cast<uint16_t*>(w + L.kc),
       vct = reinterpret_cast<uint16_t*>(w + L.vct);
  int* plan = plan_out ? plan_out : reinterpret_cast<int*>(w + L.plan);
  hipError_t e = wf_launch("wf_vsa_gather", s, [&] {
    hipLaunchKernelGGL((wf_vsa_gather<128, 0>), dim3((unsigned)(BH * g.C)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), qc, kc, vct, reinterpret_cast<float*>(w + L.qbar),
                       reinterpret_cast<float*>(w + L.kbar), reinterpret_cast<uint16_t*>(w + L.vbt), g, 0.0);
  });
  if (e != hipSuccess) return e;
  e = wf_launch("wf_sta_plan", s, [&] {
    hipLaunchKernelGGL(wf_sta_plan, dim3((unsigned)(((long)g.C * kk + 255) / 256)), dim3(256), 0, s, plan, g,
                       wt, wh, ww);
  });
  if (e != hipSuccess) return e;
  return wf_launch("wf_sta_fine", s, [&] {
    hipLaunchKernelGGL((wf_vsa_fine_fwd<128, false, kSoftmaxGuarded>), dim3((unsigned)(BH * g.C)), dim3(128), 0, s,
                       qc, kc, vct, plan, o, lse, nullptr, nullptr, g, kk, 0L, scale * kLog2e);
  });
}

hipError_t launch_vsa_fine_gated(void* ws, const int* idx, const void* gate, int BH, int T, int H,
                                 int W, int D, float scale, int topk, float* o, float* lse,
                                 float* o_coarse, hipStream_t s) {
  const Grid3 g = make_grid(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  float* oc = o_coarse ? o_coarse : reinterpret_cast<float*>(w + L.ocoarse);
  const int rblocks = (g.C + 31) / 32;
  hipError_t e = wf_launch("wf_vsa_coarse_out", s, [&] {
    hipLaunchKernelGGL(wf_vsa_coarse_out<128>, dim3((unsigned)(BH * rblocks)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(w + L.scores),
                       reinterpret_cast<const float2*>(w + L.stat),
                       reinterpret_cast<const uint16_t*>(w + L.vbt), oc, g.C, g.Cs, rblocks);
  });
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
