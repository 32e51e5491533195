// Dense bidirectional self-attention over the token grid, bf16 MFMA on gfx950.
//
// Operation: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "Why
// video attention becomes the bottleneck": every query against every key of
// the grid, O = softmax(scale Q K^T) V per (batch, head), computed tile by tile
// without materialising the score matrix; the softmax keeps a running row
// maximum (section "Fixed-max softmax is a numerical contract").
#include "wf_device.hpp"
#include "wf_launch.hpp"

namespace wf {

// V [BH][N][D] -> V^T [BH][D][Np] (Np = N rounded up to 64), keys in perm16
// order inside each group of 16, zero columns for keys >= N.  One workgroup
// per (bh, 64-key block), through an LDS tile.
template <int D>
__global__ void __launch_bounds__(256) wf_transpose_v(const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ vt, int N, int Np) {
  constexpr int STR = D + 2;  // odd word stride: column reads hit distinct banks
  __shared__ uint16_t tile[64 * STR];
  const int nblk = Np / 64;
  const int bh = blockIdx.x / nblk, n0 = (blockIdx.x % nblk) * 64, tid = threadIdx.x;
  const uint16_t* src = v + ((long)bh * N + n0) * D;
  constexpr int ROWCH = D / 8;
  for (int id = tid; id < 64 * ROWCH; id += 256) {
    const int r = id / ROWCH, c = id % ROWCH;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (n0 + r < N) u = *reinterpret_cast<const uint4*>(src + (long)r * D + c * 8);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&u);
#pragma unroll
    for (int t = 0; t < 8; ++t) tile[r * STR + c * 8 + t] = e[t];
  }
  __syncthreads();
  uint16_t* dst = vt + (long)bh * D * Np + n0;
  for (int id = tid; id < D * 8; id += 256) {
    const int d = id / 8, pc = id % 8;  // output positions 8*pc .. 8*pc+7 of row d
    uint16_t e[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) e[t] = tile[perm16(pc * 8 + t) * STR + d];
    *reinterpret_cast<uint4*>(dst + (long)d * Np + pc * 8) = *reinterpret_cast<const uint4*>(e);
  }
}

// ---------------------------------------------------------------------------
// Ping-pong dense kernel: 8 wavefronts (2 per SIMD) x 32 query rows = 256 rows
// per workgroup.  Every wavefront alternates an MFMA phase (P(t-1) V(t-1) then
// S(t) = K(t) Q^T) and a VALU phase (softmax of S(t)).  Half B runs one
// barrier behind half A, so on every SIMD one wavefront is in its MFMA phase
// while the other is in its VALU phase.  K(t) and V(t-1) are resident during
// global phases 2t and 2t+1; in its VALU phase t half A copies K(t+1) and V(t)
// global -> LDS directly (no staging registers) into the slots that K(t-1)
// and V(t-2) left, and waits for them before the phase's closing barrier.
// Within an MFMA phase the LDS operand reads run four MFMAs ahead of use.
template <int D>
__global__ void __launch_bounds__(512, 1)
wf_dense_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
             int N, int Np, int nqt, float sl2) {
  constexpr int DB = D / 32;
  __shared__ __align__(16) char kt0[Swz<D>::KB];
  __shared__ __align__(16) char kt1[Swz<D>::KB];
  __shared__ __align__(16) char vt0[Swz<D>::VB];
  __shared__ __align__(16) char vt1[Swz<D>::VB];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, j = lane % 32, half = lane / 32;
  const bool isB = wave >= 4;
  const int wq = wave & 3;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nqt, qt = item % nqt;
  const long base = (long)bh * N;
  const uint16_t* kg = k + base * D;
  const uint16_t* vg = vt + (long)bh * D * Np;
  const int qrow = qt * 256 + wave * 32 + j;

  bf16x8 qop[D / 16];
  {
    const uint16_t* qr = q + (base + min(qrow, N - 1)) * D;
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
#pragma unroll
  for (int i = 0; i < 16; ++i) p2[i] = (bf16x2){(__bf16)0.f, (__bf16)0.f};
  // the first MFMA phase runs P V on zero probabilities: give it a zero V slot too
  for (int i = tid; i < Swz<D>::VB / 16; i += 512) reinterpret_cast<uint4*>(vt1)[i] = make_uint4(0, 0, 0, 0);

  const int nt = (N + 63) / 64;
  if (!isB) {
    tile_copy<D, 4>(kg, N, kt0, nullptr, 0, nullptr, wq, lane);
    wait_tile_copies();
  }
  __syncthreads();
  if (isB) __syncthreads();  // half B runs one phase behind

  // one MFMA phase and one VALU phase for tile t; kcur = K(t), vprev = V(t-1),
  // knext / vfill receive K(t+1) / V(t)
  auto phase_pair = [&](int t, const char* kcur, const char* vprev, char* knext, char* vfill) {
    // Uniform MFMA phase: at t = 0 the probabilities are zero; at t = nt the scores come
    // from stale (finite) K data and are never used.
    __builtin_amdgcn_sched_barrier(0);
    mfma_run<D, 0, Pairs<D>::NPV + Pairs<D>::NQK>(vprev, kcur, p2, qop, oacc, s0, s1, j, half);
    __syncthreads();
    if (!isB && t < nt)
      tile_copy<D, 4>(t + 1 < nt ? kg + (long)(t + 1) * 64 * D : nullptr, N - (t + 1) * 64, knext,
                      vg + (long)t * 64, Np, vfill, wq, lane);
    if (t < nt) {
      if ((t + 1) * 64 > N) {  // ragged last tile: keys >= N do not exist
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (t * 64 + key_row(0, r, half) >= N) s0[r] = -INFINITY;
          if (t * 64 + key_row(1, r, half) >= N) s1[r] = -INFINITY;
        }
      }
      softmax_tile<DB>(s0, s1, sl2, m, l, oacc, p2);
    }
    if (!isB) wait_tile_copies();
    __syncthreads();
  };
  // tiles alternate between the two K slots and the two V slots; unrolled by two so
  // every LDS array is named statically (keeps the compiler's LDS alias tracking exact)
  for (int t = 0; t <= nt; t += 2) {
    phase_pair(t, kt0, vt1, kt1, vt0);
    if (t + 1 <= nt) phase_pair(t + 1, kt1, vt0, kt0, vt1);
  }
  if (!isB) __syncthreads();  // same barrier count in both halves

  const float lse_row = finish_store<DB>(oacc, m, l, qrow < N ? o + (base + qrow) * D : nullptr, half);
  if (lse && qrow < N && half == 0) lse[base + qrow] = lse_row;
}

template <int D>
static hipError_t launch_dense_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                                 float* lse, int BH, int N, float scale, uint16_t* vt,
                                 hipStream_t s) {
  const int Np = (N + 63) / 64 * 64;
  hipError_t e = wf_launch("wf_transpose_v", s, [&] {
    hipLaunchKernelGGL(wf_transpose_v<D>, dim3((unsigned)((long)(Np / 64) * BH)), dim3(256), 0, s, v, vt,
                       N, Np);
  });
  if (e != hipSuccess) return e;
  const int nqt = (N + 255) / 256;
  const long grid = (long)nqt * BH;
  return wf_launch("wf_dense_fwd", s, [&] {
    hipLaunchKernelGGL((wf_dense_fwd<D>), dim3((unsigned)grid), dim3(512), 0, s,
                       q, k, vt, o, lse, N, Np, nqt, scale * kLog2e);
  });
}

size_t dense_workspace_bytes(int BH, int N, int D) {
  const long Np = ((long)N + 63) / 64 * 64;
  return (size_t)BH * D * Np * 2;
}

hipError_t launch_dense(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                        int N, int D, float scale, void* ws, hipStream_t s) {
  auto q16 = static_cast<const uint16_t*>(q), k16 = static_cast<const uint16_t*>(k),
       v16 = static_cast<const uint16_t*>(v);
  auto vt = static_cast<uint16_t*>(ws);
  if (D == 128) return launch_dense_d<128>(q16, k16, v16, o, lse, BH, N, scale, vt, s);
  return launch_dense_d<64>(q16, k16, v16, o, lse, BH, N, scale, vt, s);
}

}  // namespace wf
