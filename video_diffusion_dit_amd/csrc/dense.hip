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
// LDS tiles are unpadded; each 16-byte chunk is XOR-swizzled within its row
// so that 16 lanes reading one chunk of 16 consecutive rows hit 16 distinct
// 16-byte bank groups (gfx950 LDS: 64 banks x 4 bytes).
template <int D>
struct PP {
  static constexpr int KB = 64 * D * 2;   // K tile bytes
  static constexpr int VB = D * 64 * 2;   // V^T tile bytes
  static constexpr int KCPR = D / 8;      // chunks per K row
  // chunk slot of (row, chunk) in a K tile / a V^T tile
  __host__ __device__ static constexpr int kslot(int r, int c) {
    return KCPR == 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
  }
  __host__ __device__ static constexpr int vslot(int d, int c) { return c ^ ((d >> 1) & 7); }
};

// Half A (4 wavefronts) copies one K tile (rows clamped to krows-1) and one V^T tile.
template <int D>
__device__ __forceinline__ void pp_copy(const uint16_t* __restrict__ kg, int krows, char* kdst,
                                        const uint16_t* __restrict__ vg, long vld, char* vdst,
                                        int wq, int lane) {
  constexpr int KPIECES = PP<D>::KB / 1024, VPIECES = PP<D>::VB / 1024, CPR = PP<D>::KCPR;
  if (kg) {
#pragma unroll
    for (int i = 0; i < KPIECES / 4; ++i) {
      const int g = i * 4 + wq, P = g * 64 + lane;
      const int r = P / CPR, slot = P % CPR;
      const int c = PP<D>::kslot(r, slot);  // the swizzle is an involution in c
      const int rr = min(r, krows - 1);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kg + (long)rr * D + c * 8),
                                       (__attribute__((address_space(3))) void*)(kdst + g * 1024), 16, 0, 0);
    }
  }
  if (vg) {
#pragma unroll
    for (int i = 0; i < VPIECES / 4; ++i) {
      const int g = i * 4 + wq, P = g * 64 + lane;
      const int d = P / 8, slot = P % 8;
      const int c = PP<D>::vslot(d, slot);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vg + (long)d * vld + c * 8),
                                       (__attribute__((address_space(3))) void*)(vdst + g * 1024), 16, 0, 0);
    }
  }
}

// The MFMA phase as 32 (LDS operand, MFMA) pairs: 16 of P V (operand = V^T rows),
// then 16 of K Q^T (operand = K rows).  Operands are loaded four pairs ahead of
// the MFMAs that consume them, in chunks fenced with sched_barrier so the
// compiler keeps the prefetch distance.
template <int D>
__device__ __forceinline__ uint4 pp_operand(int i, const char* vt, const char* kt, int j, int half) {
  constexpr int NPV = 4 * (D / 32);
  if (i < NPV) {  // PV: ks = i / DB, b = i % DB
    const int ks = i / (D / 32), b = i % (D / 32), d = b * 32 + j, c = ks * 2 + half;
    return *reinterpret_cast<const uint4*>(vt + d * 128 + PP<D>::vslot(d, c) * 16);
  }
  const int kk = (i - NPV) / 2, r = ((i - NPV) % 2) * 32 + j, c = kk * 2 + half;
  return *reinterpret_cast<const uint4*>(kt + r * (D * 2) + PP<D>::kslot(r, c) * 16);
}

template <int D>
__device__ __forceinline__ void pp_mfma(int i, uint4 a, const bf16x2* p2, const bf16x8* qop, f32x16* o,
                                        f32x16& s0, f32x16& s1) {
  constexpr int NPV = 4 * (D / 32);
  if (i < NPV) {
    const int ks = i / (D / 32), b = i % (D / 32);
    const int base = (ks / 2) * 8 + (ks % 2) * 4;
    const bf16x8 p = __builtin_bit_cast(bf16x8, P4{p2[base], p2[base + 1], p2[base + 2], p2[base + 3]});
    o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), p, o[b], 0, 0, 0);
  } else {
    const int kk = (i - NPV) / 2;
    if ((i - NPV) % 2 == 0) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qop[kk], s0, 0, 0, 0);
    else s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qop[kk], s1, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void pp_mfma_phase(const char* vt, const char* kt, const bf16x2* p2,
                                              const bf16x8* qop, f32x16* o, f32x16& s0, f32x16& s1,
                                              int j, int half) {

  constexpr int NP = 4 * (D / 32) + 2 * (D / 16), PF = 4, R = PF + 1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
  uint4 ring[R];
#pragma unroll
  for (int u = 0; u < PF; ++u) ring[u] = pp_operand<D>(u, vt, kt, j, half);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (i + PF < NP) ring[(i + PF) % R] = pp_operand<D>(i + PF, vt, kt, j, half);
    pp_mfma<D>(i, ring[i % R], p2, qop, o, s0, s1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__global__ void __launch_bounds__(512, 1)
wf_dense_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
             int N, int Np, int nqt, float sl2) {
  constexpr int DB = D / 32;
  __shared__ __align__(16) char kt0[PP<D>::KB];
  __shared__ __align__(16) char kt1[PP<D>::KB];
  __shared__ __align__(16) char vt0[PP<D>::VB];
  __shared__ __align__(16) char vt1[PP<D>::VB];
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
  for (int i = tid; i < PP<D>::VB / 16; i += 512) reinterpret_cast<uint4*>(vt1)[i] = make_uint4(0, 0, 0, 0);

  const int nt = (N + 63) / 64;
  if (!isB) {
    pp_copy<D>(kg, N, kt0, nullptr, 0, nullptr, wq, lane);
    wait_tile_copies();
  }
  __syncthreads();
  if (isB) __syncthreads();  // half B runs one phase behind

  auto mfma_phase = [&](int t, const char* kcur, const char* vprev, char* knext, char* vfill) {
    // uniform phase: at t = 0 the probabilities are zero (and the V slot zeroed); at t = nt the
    // scores come from stale (finite) K data and are never used
    __builtin_amdgcn_sched_barrier(0);
    pp_mfma_phase<D>(vprev, kcur, p2, qop, oacc, s0, s1, j, half);
    __syncthreads();
  };
  auto valu_phase = [&](int t, char* knext, char* vfill) {
    if (!isB && t < nt)
      pp_copy<D>(t + 1 < nt ? kg + (long)(t + 1) * 64 * D : nullptr, N - (t + 1) * 64, knext,
                 vg + (long)t * 64, Np, vfill, wq, lane);
    if (t < nt) {
      if ((t + 1) * 64 > N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (t * 64 + key_row(0, r, half) >= N) s0[r] = -INFINITY;
          if (t * 64 + key_row(1, r, half) >= N) s1[r] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
      mx = wave_max_pair(mx) * sl2;
      if (__ballot(mx > m + kLazy)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      }
      const float nm = -m;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p2[r] = __builtin_convertvector(
            (f32x2){__builtin_amdgcn_exp2f(__builtin_fmaf(s0[2 * r], sl2, nm)),
                    __builtin_amdgcn_exp2f(__builtin_fmaf(s0[2 * r + 1], sl2, nm))}, bf16x2);
        p2[8 + r] = __builtin_convertvector(
            (f32x2){__builtin_amdgcn_exp2f(__builtin_fmaf(s1[2 * r], sl2, nm)),
                    __builtin_amdgcn_exp2f(__builtin_fmaf(s1[2 * r + 1], sl2, nm))}, bf16x2);
      }
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        la = __builtin_amdgcn_fdot2_f32_bf16(p2[i], one2, la, false);
        lb = __builtin_amdgcn_fdot2_f32_bf16(p2[i + 1], one2, lb, false);
      }
      l += la + lb;
    }
    if (!isB) wait_tile_copies();
    __syncthreads();
  };
  // tiles alternate between the two K slots and the two V slots; unrolled by two so
  // every LDS array is named statically
  for (int t = 0; t <= nt; t += 2) {
    mfma_phase(t, kt0, vt1, kt1, vt0);
    valu_phase(t, kt1, vt0);
    if (t + 1 <= nt) {
      mfma_phase(t + 1, kt1, vt0, kt0, vt1);
      valu_phase(t + 1, kt0, vt1);
    }
  }
  if (!isB) __syncthreads();  // same barrier count in both halves

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  if (qrow < N) {
    float* orow = o + (base + qrow) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(orow + b * 32 + rq * 8 + half * 4) =
            make_float4(oacc[b][rq * 4] * inv, oacc[b][rq * 4 + 1] * inv, oacc[b][rq * 4 + 2] * inv,
                        oacc[b][rq * 4 + 3] * inv);
    if (lse && half == 0) lse[base + qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
  }
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
