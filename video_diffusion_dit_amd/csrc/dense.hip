// Dense bidirectional self-attention over the token grid, bf16 MFMA on gfx950.
//
// Operation: "Anatomy of Wan2.2's 53.6x speedup" (zharfai.com), section "Why
// video attention becomes the bottleneck": every query against every key of
// the grid, O = softmax(scale Q K^T) V per (batch, head), computed tile by tile
// without materialising the score matrix; the softmax keeps a running row
// maximum (section "Fixed-max softmax is a numerical contract").
#include <type_traits>

#include "wf_device.hpp"
#include "wf_launch.hpp"

namespace wf {

// V [BH][N][D] -> V^T tiles [BH][Np/64][D][64] (Np = N rounded up to 64): each
// 64-key block of a head transposed into one contiguous D x 64 tile, keys in
// perm16 order inside each group of 16, zero columns for keys >= N.  One
// workgroup per (bh, 64-key block), through an LDS tile.
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
  uint16_t* dst = vt + ((long)bh * Np + n0) * D;  // this block's tile
  for (int id = tid; id < D * 8; id += 256) {
    const int d = id / 8, pc = id % 8;  // output positions 8*pc .. 8*pc+7 of row d
    uint16_t e[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) e[t] = tile[perm16(pc * 8 + t) * STR + d];
    *reinterpret_cast<uint4*>(dst + d * 64 + pc * 8) = *reinterpret_cast<const uint4*>(e);
  }
}

// ---------------------------------------------------------------------------
// Ping-pong dense kernel: 8 wavefronts (2 per SIMD) x 32 query rows = 256 rows
// per workgroup.  Every wavefront alternates an MFMA phase (P(t-1) V(t-1) then
// S(t) = K(t) Q^T) and a VALU phase (softmax of S(t)).  Half B runs one
// barrier behind half A, so on every SIMD one wavefront is in its MFMA phase
// (at raised issue priority) while the other is in its VALU phase.  K and V^T
// tiles rotate through three LDS slots each, filled global -> LDS with buffer
// loads (no staging registers): in its VALU phase t half A copies K(t+2) into
// the slot K(t-1) left and half B copies V(t+2) into the slot V(t-1) left, so
// the copy work is split evenly over the two halves; each waits for its copies
// at the end of its next MFMA phase, so each copy has a phase to land.  Within an MFMA phase the
// LDS operand reads run four MFMAs ahead of use, at offsets precomputed once per workgroup
// (OperandTable: 12 registers that save an address computation per read); the first four are read early in
// the wavefront's VALU phase, right after its copies, so their latency hides behind the
// softmax.  SM selects the
// softmax reference policy (softmax_tile; the library default is the guarded
// integer reference).
template <int D, int SM>
__global__ void __launch_bounds__(512, 1)
wf_dense_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
             int N, int Np, int nqt, float sl2) {
  constexpr int DB = D / 32;
  __shared__ __align__(16) char kt0[Swz<D>::KB];
  __shared__ __align__(16) char kt1[Swz<D>::KB];
  __shared__ __align__(16) char kt2[Swz<D>::KB];
  __shared__ __align__(16) char vt0[Swz<D>::VB];
  __shared__ __align__(16) char vt1[Swz<D>::VB];
  __shared__ __align__(16) char vt2[Swz<D>::VB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, j = lane % 32,
            half = lane / 32;
  const bool isB = wave >= 4;
  const int wq = __builtin_amdgcn_readfirstlane(wave & 3);
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nqt, qt = item % nqt;
  const long base = (long)bh * N;
  const uint16_t* kg = k + base * D;
  const uint16_t* vg = vt + (long)bh * D * Np;  // the head's V^T tiles, tile t at vg + t * 64 * D
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
  for (int i = tid; i < Swz<D>::VB / 16; i += 512) reinterpret_cast<uint4*>(vt2)[i] = make_uint4(0, 0, 0, 0);

  const int nt = (N + 63) / 64;
  // Three K slots and three V slots: tile t's K sits in slot t % 3, its V in slot t % 3.
  // Prologue: K(0), K(1) and V(0) by half A, V(1) by half B.
  const CopyOffsets<D, 4> coff(wq, lane, 64);  // V^T tile rows are 64 keys apart
  constexpr uint32_t VTB = Swz<D>::VB;           // bytes of one V^T tile
  if (!isB) {
    tile_copy<D, 4>(coff, kg, N, kt0, nullptr, 0, 0, nullptr, wq);
    tile_copy<D, 4>(coff, nt > 1 ? kg + 64 * D : nullptr, N - 64, kt1, vg, 64, VTB, vt0, wq);
  } else {
    tile_copy<D, 4>(coff, nullptr, 0, nullptr, vg + 64 * D, 64, nt > 1 ? VTB : 0u, vt1, wq);
  }
  __syncthreads();  // its fence waits for all four copies
  if (isB) __syncthreads();  // half B runs one phase behind

  // one MFMA phase and one VALU phase for tile t; kcur = K(t), vprev = V(t-1).  With half A's
  // MFMA phase t in global phase 2t and its VALU phase t in 2t+1 (half B one phase later):
  //   - half A copies K(t+2) into knext, the slot K(t-1) left, in its VALU phase (2t+1),
  //     waits for it at the end of its MFMA phase t+1 (2t+2) and so publishes it from 2t+3;
  //     K(t+2) is first read in 2t+4;
  //   - half B copies V(t+2) into vprev's slot, V(t-1), which both halves finished reading in
  //     their MFMA phases t, in its VALU phase (2t+2), waits at the end of its MFMA phase t+1
  //     (2t+3) and publishes it from 2t+4; V(t+2) is first read by half A's operand prefetch
  //     at the end of 2t+5.
  // So each copy has one full phase to land, and both halves issue 4 copies per VALU phase.
  // The first operands of every MFMA phase are read at the start of the wavefront's previous
  // VALU phase (V(t) was published by the barrier that opened it), so the matrix pipe does not
  // idle through the LDS latency at each phase start and the reads overlap the softmax.
  uint4 ring[kRing];
  const OperandTable<D, false> otab(j, half);  // every operand read's LDS offset
  auto phase_pair = [&](auto half_a_c, int t, const char* kcur, const char* vprev, char* knext,
                        const char* vnext) __attribute__((always_inline)) {
    constexpr bool HALF_A = decltype(half_a_c)::value;  // half A copies K tiles, half B V^T tiles
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);  // MFMA phase first at the SIMD's issue arbiter
    mfma_run<D, 0, Pairs<D>::NPV + Pairs<D>::NQK, true>(vprev, kcur, p2, qop, oacc, s0, s1, otab, ring);
    __builtin_amdgcn_s_setprio(0);
    wait_tile_copies();  // half A: K(t+1) landed; half B: V(t+1) landed
    barrier_nofence();
    // Always 4 copy instructions per wavefront: a tile past the end gets a zero-length
    // descriptor (no memory access) into a slot nobody reads again.  Half A copies K(t+2) into
    // K(t-1)'s slot; half B, one phase later, copies V(t+2) into V(t-1)'s slot, which both
    // halves finished reading in their MFMA phases t.
    if constexpr (HALF_A)
      tile_copy<D, 4>(coff, kg + (long)(t + 2) * 64 * D, N - (t + 2) * 64, knext, nullptr, 0, 0u, nullptr, wq);
    else
      tile_copy<D, 4>(coff, nullptr, 0, nullptr, vg + (long)(t + 2) * 64 * D, 64, t + 2 < nt ? VTB : 0u,
                      const_cast<char*>(vprev), wq);
    mfma_prefill<D, 0>(ring, vnext, kcur, otab);  // first operands of MFMA phase t+1: V(t) rows
    if (t < nt) {
      if ((t + 1) * 64 > N) {  // ragged last tile: keys >= N do not exist
        // selects that read the scores: a plain store into an MFMA result register is not
        // ordered against the MFMA's own write-back, a read waits for it
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = t * 64 + key_row(0, r, half) < N ? s0[r] : -INFINITY;
          s1[r] = t * 64 + key_row(1, r, half) < N ? s1[r] : -INFINITY;
        }
      }
      softmax_tile<DB, SM>(s0, s1, sl2, m, l, oacc, p2);
    }
    barrier_nofence();
  };
  // unrolled by three so every LDS array is named statically, and instantiated once per half
  // (half A or B) so the compiler tracks the copies on straight-line paths
  auto tile_loop = [&](auto half_a_c) __attribute__((always_inline)) {
    mfma_prefill<D, 0>(ring, vt2, kt0, otab);  // MFMA phase 0: V(-1), the zero slot
    for (int t = 0; t <= nt; t += 3) {
      phase_pair(half_a_c, t, kt0, vt2, kt2, vt0);
      if (t + 1 <= nt) {  // nested, so every path into a phase passes the previous phase's wait
        phase_pair(half_a_c, t + 1, kt1, vt0, kt0, vt1);
        if (t + 2 <= nt) phase_pair(half_a_c, t + 2, kt2, vt1, kt1, vt2);
      }
    }
  };
  if (!isB) tile_loop(std::true_type());
  else tile_loop(std::false_type());
  wait_tile_copies();          // no copy may still be writing LDS when the workgroup ends
  if (!isB) barrier_nofence();  // same barrier count in both halves

  const float lse_row = finish_store<DB>(oacc, m, l, qrow < N ? o + (base + qrow) * D : nullptr, half);
  if (lse && qrow < N && half == 0) lse[base + qrow] = lse_row;
}

template <int D>
static hipError_t launch_dense_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                                 float* lse, int BH, int N, float scale, int softmax_mode, uint16_t* vt,
                                 hipStream_t s) {
  const int Np = (N + 63) / 64 * 64;
  hipError_t e = wf_launch("wf_transpose_v", s, [&] {
    hipLaunchKernelGGL(wf_transpose_v<D>, dim3((unsigned)((long)(Np / 64) * BH)), dim3(256), 0, s, v, vt,
                       N, Np);
  });
  if (e != hipSuccess) return e;
  const int nqt = (N + 255) / 256;
  const long grid = (long)nqt * BH;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(512), 0, s, q, k, vt, o, lse, N, Np, nqt, scale * kLog2e);
  };
  if (softmax_mode == kSoftmaxRunningMax)
    return wf_launch("wf_dense_fwd_running_max", s, [&] { go(wf_dense_fwd<D, kSoftmaxRunningMax>); });
  if (softmax_mode == kSoftmaxFixedFirst)
    return wf_launch("wf_dense_fwd_fixed_first", s, [&] { go(wf_dense_fwd<D, kSoftmaxFixedFirst>); });
  return wf_launch("wf_dense_fwd", s, [&] { go(wf_dense_fwd<D, kSoftmaxGuarded>); });
}

size_t dense_workspace_bytes(int BH, int N, int D) {
  const long Np = ((long)N + 63) / 64 * 64;
  return (size_t)BH * D * Np * 2;
}

hipError_t launch_dense(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                        int N, int D, float scale, int softmax_mode, void* ws, hipStream_t s) {
  auto q16 = static_cast<const uint16_t*>(q), k16 = static_cast<const uint16_t*>(k),
       v16 = static_cast<const uint16_t*>(v);
  auto vt = static_cast<uint16_t*>(ws);
  if (D == 128) return launch_dense_d<128>(q16, k16, v16, o, lse, BH, N, scale, softmax_mode, vt, s);
  return launch_dense_d<64>(q16, k16, v16, o, lse, BH, N, scale, softmax_mode, vt, s);
}

}  // namespace wf
