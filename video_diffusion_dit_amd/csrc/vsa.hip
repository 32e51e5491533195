// Video Sparse Attention (VSA) on gfx950: cube gather and pooling, coarse
// cube scores, per-cube top-k and fine block-sparse attention.
//
// Operation: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "VSA
// selects cubes": pad the T x H x W grid to multiples of 4, cut it into 4x4x4
// cubes of 64 tokens, score cube-mean queries against cube-mean keys, keep the
// top-k key cubes of every query cube, then run token-level attention of each
// query cube over those cubes only.  Section "Roofline analysis set the 3.35
// ms target" counts one output tile per (query cube, head).
#include "wf_device.hpp"
#include "wf_launch.hpp"

namespace wf {

struct Grid3 {
  int T, H, W, nt, nh, nw, C;
};

static Grid3 make_grid(int T, int H, int W) {
  Grid3 g{T, H, W, (T + 3) / 4, (H + 3) / 4, (W + 3) / 4, 0};
  g.C = g.nt * g.nh * g.nw;
  return g;
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
// zero), Vct [BH][C][D][64] (slots in perm16 order) and the fp32 means of Q and
// K over the cube's real tokens.
template <int D>
__global__ void __launch_bounds__(256) wf_vsa_gather(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qc, uint16_t* __restrict__ kc, uint16_t* __restrict__ vct,
    float* __restrict__ qbar, float* __restrict__ kbar, Grid3 g) {
  constexpr int ROWCH = D / 8;            // 16-byte chunks per row
  constexpr int RSTEP = 256 / ROWCH;      // rows covered by one pass of the workgroup
  constexpr int VSTR = D + 2;
  __shared__ float red[RSTEP][D];
  __shared__ uint16_t vtile[64 * VSTR];
  const int tid = threadIdx.x, c16 = tid % ROWCH, r0 = tid / ROWCH;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.C, c = item % g.C;
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
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
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&u);
      if (which < 2) {
        uint16_t* dst = (which == 0 ? qc : kc) + (cube_row0 + s) * D + c16 * 8;
        *reinterpret_cast<uint4*>(dst) = u;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += __uint_as_float((uint32_t)e[t] << 16);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) vtile[s * VSTR + c16 * 8 + t] = e[t];
      }
    }
    if (which < 2) {
#pragma unroll
      for (int t = 0; t < 8; ++t) red[r0][c16 * 8 + t] = acc[t];
      __syncthreads();
      if (tid < D) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RSTEP; ++r) sum += red[r][tid];
        float* dst = (which == 0 ? qbar : kbar) + ((long)bh * g.C + c) * D;
        dst[tid] = sum / (float)count;
      }
      __syncthreads();
    } else {
      __syncthreads();
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
// S[bh][c][c'] = scale * sum_d Qbar[c][d] Kbar[c'][d] in fp32; 64x64 output
// tile per workgroup, 4x4 per thread.
template <int D>
__global__ void __launch_bounds__(256) wf_vsa_scores(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar,
                                                     float* __restrict__ s, int C, int ntile,
                                                     float scale) {
  constexpr int DK = 32;
  __shared__ float As[DK][64 + 4];
  __shared__ float Bs[DK][64 + 4];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int per_head = ntile * ntile;
  const int bh = blockIdx.x / per_head, rem = blockIdx.x % per_head;
  const int r0 = (rem / ntile) * 64, c0 = (rem % ntile) * 64;
  const float* A = qbar + (long)bh * C * D;
  const float* Bm = kbar + (long)bh * C * D;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += DK) {
    for (int id = tid; id < 64 * DK; id += 256) {
      const int r = id / DK, dd = id % DK;
      As[dd][r] = (r0 + r < C) ? A[(long)(r0 + r) * D + d0 + dd] : 0.f;
      Bs[dd][r] = (c0 + r < C) ? Bm[(long)(c0 + r) * D + d0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < DK; ++dd) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[dd][ty * 4 + i]; b[i] = Bs[dd][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = __builtin_fmaf(a[i], b[jj], acc[i][jj]);
    }
    __syncthreads();
  }
  float* out = s + (long)bh * C * C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty * 4 + i;
    if (r >= C) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int cc = c0 + tx * 4 + jj;
      if (cc < C) out[(long)r * C + cc] = acc[i][jj] * scale;
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wavefront per score row.  Lane L holds candidates c' = e*64 + L.  The
// k-th largest order key is found bit by bit (count of keys >= candidate via
// ballots); keys above it are all kept, keys equal to it are kept in
// ascending c' order until k are chosen.  Output is ascending.
template <int E>
__global__ void __launch_bounds__(256) wf_vsa_topk(const float* __restrict__ s,
                                                   int* __restrict__ idx, long rows, int C,
                                                   int k) {
  const int lane = threadIdx.x % 64;
  const long row = (long)blockIdx.x * 4 + threadIdx.x / 64;
  if (row >= rows) return;
  const float* sr = s + row * C;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int cc = e * 64 + lane;
    key[e] = cc < C ? order_key(sr[cc]) : 0u;
  }
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
// scattered back to grid order, padded query slots are not written.
template <int D>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) wf_vsa_fine_fwd(
    const uint16_t* __restrict__ qc, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vct, const int* __restrict__ idx, float* __restrict__ o,
    float* __restrict__ lse, Grid3 g, int k, float sl2) {
  constexpr int DB = D / 32, NPV = Pairs<D>::NPV, NQK = Pairs<D>::NQK;
  __shared__ __align__(16) char ks[Swz<D>::KB];
  __shared__ __align__(16) char vs[Swz<D>::VB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, j = lane % 32,
            half = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.C, c = item % g.C;
  const long cube_base = (long)bh * g.C;
  const int* plan = idx + ((long)bh * g.C + c) * k;
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
    softmax_tile<DB>(s0, s1, sl2, m, l, oacc, p2);
    wait_tile_copies_keep<KP>();  // V(t) landed (it had the scores and the softmax to do so); K(t+1) may fly
    barrier_nofence();            // V(t) visible
    mfma_run<D, 0, NPV>(vs, ks, p2, qop, oacc, s0, s1, j, half);  // O += P V(t)
    barrier_nofence();                                             // V slot free
    tile_copy<D, 2>(coff, nullptr, 0, nullptr, vct + (cube_base + nxt) * D * 64, 64, CUBE_BYTES, vs, wave);
    wait_tile_copies_keep<VP>();  // K(t+1) landed; V(t+1) may fly
    cur = nxt;
  }
  wait_tile_copies();  // no copy may still be writing LDS when the workgroup ends
  int ct, ch, cw;
  cube_coords(g, c, ct, ch, cw);
  const int tok = slot_token(g, ct, ch, cw, slot);
  const long row = (long)bh * g.T * g.H * g.W + tok;
  const float lse_row = finish_store<DB>(oacc, m, l, tok >= 0 ? o + row * D : nullptr, half);
  if (lse && tok >= 0 && half == 0) lse[row] = lse_row;
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
  L.scores = L.kbar + up((size_t)BH * g.C * D * 4);
  L.flag = L.scores + up((size_t)BH * g.C * g.C * 4);
  L.total = L.flag + 256;
  return L;
}

hipError_t launch_vsa_coarse(const void* q, const void* k, const void* v, int BH, int T, int H,
                             int W, int D, float scale, int topk, int* idx, float* scores_out,
                             void* ws, hipStream_t s) {
  const Grid3 g = make_grid(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  char* w = static_cast<char*>(ws);
  auto qc = reinterpret_cast<uint16_t*>(w + L.qc), kc = reinterpret_cast<uint16_t*>(w + L.kc),
       vct = reinterpret_cast<uint16_t*>(w + L.vct);
  auto qbar = reinterpret_cast<float*>(w + L.qbar), kbar = reinterpret_cast<float*>(w + L.kbar);
  float* sc = scores_out ? scores_out : reinterpret_cast<float*>(w + L.scores);
  hipError_t e = wf_launch("wf_vsa_gather", s, [&] {
    hipLaunchKernelGGL(wf_vsa_gather<128>, dim3((unsigned)(BH * g.C)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), qc, kc, vct, qbar, kbar, g);
  });
  if (e != hipSuccess) return e;
  const int nt = (g.C + 63) / 64;
  e = wf_launch("wf_vsa_scores", s, [&] {
    hipLaunchKernelGGL(wf_vsa_scores<128>, dim3((unsigned)(BH * nt * nt)), dim3(256), 0, s, qbar,
                       kbar, sc, g.C, nt, scale);
  });
  if (e != hipSuccess) return e;
  const long rows = (long)BH * g.C;
  const dim3 grid((unsigned)((rows + 3) / 4));
  return wf_launch("wf_vsa_topk", s, [&] {
    if (g.C <= 1024)
      hipLaunchKernelGGL(wf_vsa_topk<16>, grid, dim3(256), 0, s, sc, idx, rows, g.C, topk);
    else if (g.C <= 2048)
      hipLaunchKernelGGL(wf_vsa_topk<32>, grid, dim3(256), 0, s, sc, idx, rows, g.C, topk);
    else
      hipLaunchKernelGGL(wf_vsa_topk<64>, grid, dim3(256), 0, s, sc, idx, rows, g.C, topk);
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
                           float scale, int topk, float* o, float* lse, hipStream_t s) {
  const Grid3 g = make_grid(T, H, W);
  const VsaLayout L = vsa_layout(BH, T, H, W, D);
  const char* w = static_cast<const char*>(ws);
  return wf_launch("wf_vsa_fine", s, [&] {
    hipLaunchKernelGGL(wf_vsa_fine_fwd<128>, dim3((unsigned)(BH * g.C)), dim3(128), 0, s, reinterpret_cast<const uint16_t*>(w + L.qc),
                       reinterpret_cast<const uint16_t*>(w + L.kc),
                       reinterpret_cast<const uint16_t*>(w + L.vct), idx, o, lse, g, topk,
                       scale * kLog2e);
  });
}

}  // namespace wf
