// Device-side building blocks shared by the dense and VSA kernels (gfx950 only).
//
// The attention tile math, per wavefront owning 32 query rows and one tile of
// 64 keys, with lane L (j = L % 32, half = L / 32):
//   S^T (64 x 32) = K_tile (64 x D) . Q^T (D x 32)      two 32x32 blocks, MFMA 32x32x16 bf16
//     A operand: K rows from LDS; B operand: Q in registers.  Lane L ends up
//     holding query j and key rows 8*(r/4) + 4*half + r%4 of each block, so a
//     query's row max / row sum only combines lanes L and L^32.
//   online softmax in the exp2 domain with a lazily raised reference max;
//   O^T (D x 32) += V^T_tile (D x 64) . P^T (64 x 32)    D/32 blocks x 4 k-steps
//     A operand: V^T rows from LDS (keys in perm16 order); B operand: the
//     probabilities straight from the score registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wf_tiles.hpp"

namespace wf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Workgroups are dispatched round-robin over the XCDs (workgroup i lands on
// XCD i % 8).  Renumber them so that each XCD receives one contiguous range of
// logical work items: consecutive items share K/V, which then stays in that
// XCD's L2.  A bijection on [0, G) for any G.
__device__ __forceinline__ int xcd_remap(int wg, int G) {
  const int q = G / kNumXcd, r = G % kNumXcd;
  const int x = wg % kNumXcd, i = wg / kNumXcd;
  return x * q + min(x, r) + i;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max_pair(float x) {  // max over lanes L and L^32
  return fmaxf(x, __shfl_xor(x, 32));
}

// Key row (0..63 inside a tile) held by register r of score block kb in lane half `half`.
__device__ __forceinline__ int key_row(int kb, int r, int half) {
  return kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
}

__device__ __forceinline__ void wait_tile_copies() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's global->LDS copies landed
}

// Workgroup barrier without __syncthreads' memory fence, whose release half
// would drain every outstanding global->LDS copy (vmcnt(0)).  The asm memory
// clobbers keep the compiler from moving LDS accesses across it; the hardware
// ordering it needs is explicit: LDS operand reads are consumed (waited) before
// a phase ends, and copies are waited with vmcnt before the barrier that
// publishes them.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// vmcnt(KEEP): every global->LDS copy of this wavefront except the KEEP most
// recently issued has landed (loads retire in issue order for this counter).
template <int KEEP>
__device__ __forceinline__ void wait_tile_copies_keep() {
  static_assert(KEEP >= 0 && KEEP < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | KEEP);
}

struct P4 {
  bf16x2 v[4];
};

// ------------------------------------------------------------------ LDS tiles
// (tile layout and copy offsets: wf_tiles.hpp)

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes
// return zero instead of touching memory (gfx9 range check on the VGPR offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane offsets of the global->LDS tile copies (CopyGeom): only KPER + 1
// per-lane offsets are kept in registers.
template <int D, int NWC>
struct CopyOffsets {
  using G = CopyGeom<D, NWC>;
  static constexpr int KPW = G::KPW, VPW = G::VPW, KPER = G::KPER;
  uint32_t k[KPER], v;
  __device__ __forceinline__ CopyOffsets(int w, int lane, int vld) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) k[i] = G::k_lane(i, w, lane);
    v = G::v_lane(w, lane, vld);
  }
};

// Copy one K tile (rows [0, krows) exist; the rest are not read and land as
// zero or stay stale, both harmless since those keys are masked) and/or one
// V^T tile (row stride vld elements, vbytes bytes addressable from vg) into
// LDS with buffer_load ... lds.  kg / vg point at the tiles' first elements;
// null skips that tile.  Every access is range-checked by the buffer
// descriptor against the extent given.
template <int D, int NWC>
__device__ __forceinline__ void tile_copy(const CopyOffsets<D, NWC>& off, const uint16_t* kg, int krows,
                                          char* kdst, const uint16_t* vg, int vld, uint32_t vbytes, char* vdst,
                                          int w) {
  using CO = CopyOffsets<D, NWC>;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  constexpr int KSTEP = CO::G::KSTEP;  // global bytes between pieces i and i + KPER
  if (kg) {  // one descriptor per KPER-piece step, bounded at row krows (scalar work only)
    const int kbytes = __builtin_amdgcn_readfirstlane(krows * D * 2);  // uniform: the clamps below stay scalar
#pragma unroll
    for (int i = 0; i < CO::KPW; ++i) {
      const int base = (i / CO::KPER) * KSTEP;
      int left = max(kbytes - base, 0);
      asm volatile("" : "+s"(left));  // SGPR: keeps the clamp off the vector unit (no v_med3 + readfirstlane)
      const uint32_t bytes = (uint32_t)min(left, KSTEP);
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(reinterpret_cast<const char*>(kg) + base, bytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(kdst + (i * NWC + w) * 1024), 16,
                                               (int)off.k[i % CO::KPER], 0, 0, 0);
    }
  }
  if (vg) {
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg, vbytes);
#pragma unroll
    for (int i = 0; i < CO::VPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(vdst + (i * NWC + w) * 1024), 16, (int)off.v,
                                               (int)CO::G::v_step(i, vld), 0, 0);
  }
}

// Copy the K tile and/or the V^T tile of key cube `cube` (K [C][64][D], V^T
// [C][D][64], one head's cube-ordered regions) into LDS.  The descriptors
// cover the head's whole region (C cubes) and the cube's byte offset goes into
// the per-lane offset, which the hardware range-checks: cube_offset maps an
// index outside [0, C) to the region's end, so a bad plan entry reads zeros
// and never touches memory outside the region.
template <int D, int NWC>
__device__ __forceinline__ void cube_copy(const CopyOffsets<D, NWC>& off, const uint16_t* khead, char* kdst,
                                          const uint16_t* vhead, char* vdst, int cube, int C, int w) {
  using CO = CopyOffsets<D, NWC>;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  constexpr uint32_t CB = 64u * D * 2;  // bytes of one cube of K (or V^T)
  const uint32_t region = (uint32_t)C * CB, at = cube_offset(cube, C, CB);
  if (khead) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(khead, region);
#pragma unroll
    for (int i = 0; i < CO::KPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(kdst + (i * NWC + w) * 1024), 16,
                                               (int)(off.k[i % CO::KPER] + at), (int)CO::G::k_step(i), 0, 0);
  }
  if (vhead) {
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vhead, region);
#pragma unroll
    for (int i = 0; i < CO::VPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(vdst + (i * NWC + w) * 1024), 16, (int)(off.v + at),
                                               (int)CO::G::v_step(i, 64), 0, 0);
  }
}

// --------------------------------------------------------- MFMA operand runs
// The MFMAs of one tile as a numbered list of (LDS operand, MFMA) pairs:
// [0, NPV) are P V (operand = V^T rows), [NPV, NPV + NQK) are K Q^T
// (operand = K rows).
template <int D>
struct Pairs {
  static constexpr int NPV = 4 * (D / 32);
  static constexpr int NQK = 2 * (D / 16);
};

// Per-lane LDS byte offsets of the MFMA operand reads.  With c = 2 s + half
// (s = k-step) the swizzled chunk is (2 s + half) ^ f(row) = 2 s ^ (half ^ f(row)),
// and the row's byte offset has zero bits where the chunk lives, so every
// operand address is one per-lane base XOR 32 s plus an immediate (the tile,
// and the 32-row block).  With VTR the V operand comes from a V tile ([keys][D],
// VtrSwz) through two transpose reads instead of one read of a V^T tile.
template <int D, bool VTR = false>
struct OperandBase {
  uint32_t k, v;
  __device__ __forceinline__ OperandBase(int j, int half) {
    const int kf = Swz<D>::KCPR == 16 ? (j & 15) : ((j >> 1) & 7);
    k = (uint32_t)(j * D * 2 + 16 * (half ^ kf));
    v = VTR ? VtrSwz::lane_base(j + 32 * half) : (uint32_t)(j * 128 + 16 * (half ^ ((j >> 1) & 7)));
  }
};

// The per-lane LDS offsets of every operand read of a tile, computed once and kept in registers
// (loop invariant; 12 registers for D = 128, 16 with VTR), so a read costs no address
// arithmetic -- 1.4% of the dense kernel's time and 1-2% of the VSA fine stage's: K k-step kk reads at k[kk] (the 32-row
// block is an immediate); a V^T read of key step ks at v[ks] (the 32-row block is an immediate),
// or, with VTR, transpose read r of dim block b at v[2 b + r] (the key step's rows are an
// immediate).
template <int D, bool VTR>
struct OperandTable {
  static constexpr int NV = VTR ? 8 : 4;
  uint32_t k[D / 16], v[NV];
  __device__ __forceinline__ OperandTable(int j, int half) {
    const OperandBase<D, VTR> ob(j, half);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k[kk] = ob.k ^ (uint32_t)(32 * kk);
#pragma unroll
    for (int x = 0; x < NV; ++x) v[x] = VTR ? (ob.v ^ (uint32_t)((4 * (x / 2) + 2 * (x % 2)) * 16)) : (ob.v ^ (uint32_t)(32 * x));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(k[kk]));
#pragma unroll
    for (int x = 0; x < NV; ++x) asm volatile("" : "+v"(v[x]));
  }
};

template <int D, bool VTR>
__device__ __forceinline__ uint4 table_operand(int i, const char* vt, const char* kt, const OperandTable<D, VTR>& tb) {
  constexpr int NPV = Pairs<D>::NPV;
  if (i < NPV) {
    const int ks = i / (D / 32), b = i % (D / 32);
    if constexpr (VTR) {
      static_assert(D == 128, "V tile rows of 256 bytes");
      typedef short s4 __attribute__((ext_vector_type(4)));
      typedef short s8 __attribute__((ext_vector_type(8)));
      typedef __attribute__((address_space(3))) s4* lds_s4;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(vt + tb.v[2 * b] + 16 * ks * 256));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(vt + tb.v[2 * b + 1] + (16 * ks + 8) * 256));
      return __builtin_bit_cast(uint4, (s8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const uint4*>(vt + b * 32 * 128 + tb.v[ks]);
    }
  }
  const int kk = (i - NPV) / 2, kb = (i - NPV) % 2;
  return *reinterpret_cast<const uint4*>(kt + kb * 32 * D * 2 + tb.k[kk]);
}

template <int D>
__device__ __forceinline__ void mfma_pair(int i, uint4 a, const bf16x2* p2, const bf16x8* qop, f32x16* o,
                                          f32x16& s0, f32x16& s1) {
  constexpr int NPV = Pairs<D>::NPV;
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

// Pairs I0, I0 + S, ... below I1 (S = 2 over the K Q^T pairs: score block s0
// only): operands are read PF pairs ahead of the MFMA that consumes
// them; each step is fenced with sched_barrier so the compiler keeps that
// distance (it otherwise reads each operand right before its MFMA and the LDS
// latency stalls the matrix pipe).  Scores are zeroed first if the run
// contains K Q^T pairs.  The ring belongs to the caller: with PREFILLED its
// first PF entries were already read by mfma_prefill (e.g. before a barrier,
// so the run starts its first MFMA without waiting for LDS).
constexpr int kRingPF = 4, kRing = kRingPF + 1;

template <int D, int I0, bool VTR>
__device__ __forceinline__ void mfma_prefill(uint4 (&ring)[kRing], const char* vt, const char* kt,
                                               const OperandTable<D, VTR>& tb) {
#pragma unroll
  for (int u = 0; u < kRingPF; ++u) ring[u] = table_operand<D, VTR>(I0 + u, vt, kt, tb);
}

template <int D, int I0, int I1, bool PREFILLED, bool VTR, int S = 1>
__device__ __forceinline__ void mfma_run(const char* vt, const char* kt, const bf16x2* p2, const bf16x8* qop,
                                           f32x16* o, f32x16& s0, f32x16& s1, const OperandTable<D, VTR>& tb,
                                           uint4 (&ring)[kRing]) {
  constexpr int PF = kRingPF, R = kRing, NP = (I1 - I0 + S - 1) / S;
  static_assert(NP >= PF, "run shorter than the prefetch distance");
  static_assert(S == 1 || (S == 2 && I0 >= Pairs<D>::NPV), "a strided run covers K Q^T pairs only");
  static_assert(!PREFILLED || S == 1, "mfma_prefill reads consecutive pairs");
  if constexpr (I1 > Pairs<D>::NPV) {
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
  }
  if constexpr (!PREFILLED) {
#pragma unroll
    for (int u = 0; u < PF; ++u) ring[u] = table_operand<D, VTR>(I0 + S * u, vt, kt, tb);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (i + PF < NP) ring[(i + PF) % R] = table_operand<D, VTR>(I0 + S * (i + PF), vt, kt, tb);
    mfma_pair<D>(I0 + S * i, ring[i % R], p2, qop, o, s0, s1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int I0, int I1, int S = 1, bool VTR>
__device__ __forceinline__ void mfma_run(const char* vt, const char* kt, const bf16x2* p2, const bf16x8* qop,
                                           f32x16* o, f32x16& s0, f32x16& s1, const OperandTable<D, VTR>& tb) {
  uint4 ring[kRing];
  mfma_run<D, I0, I1, false, VTR, S>(vt, kt, p2, qop, o, s0, s1, tb, ring);
}

// ------------------------------------------------------------- softmax tile
// Probabilities of one tile against the reference m: p = 2^(s*sl2 - m) in bf16
// (two per register, score-register order); returns this lane's sum of them.
__device__ __forceinline__ float tile_probs(const f32x16& s0, const f32x16& s1, float sl2, float m, bf16x2* p2) {
  const float nm = -m;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p2[r] = __builtin_convertvector((f32x2){__builtin_amdgcn_exp2f(__builtin_fmaf(s0[2 * r], sl2, nm)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(s0[2 * r + 1], sl2, nm))},
                                    bf16x2);
    p2[8 + r] = __builtin_convertvector((f32x2){__builtin_amdgcn_exp2f(__builtin_fmaf(s1[2 * r], sl2, nm)),
                                                __builtin_amdgcn_exp2f(__builtin_fmaf(s1[2 * r + 1], sl2, nm))},
                                        bf16x2);
  }
  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    la = __builtin_amdgcn_fdot2_f32_bf16(p2[i], one2, la, false);
    lb = __builtin_amdgcn_fdot2_f32_bf16(p2[i + 1], one2, lb, false);
  }
  return la + lb;
}

// Online softmax step for one tile of scores s0 / s1 (masked entries -inf).
// bf16 shares fp32's exponent range, so probabilities may exceed 1 (the
// reference m may lag behind the row maximum) without loss: a lane's tile sum
// is allowed up to 2^16, which keeps O and l (fp32) far from overflow for any
// |V| below 2^100.  The common path therefore skips the row max: it
// exponentiates against the current reference and checks the lane's
// probability sum.  Only when that sum exceeds 2^16 (or is inf / NaN) -- or
// on the first tile, when m is still -inf -- does it take the row max, raise
// m, rescale O and l, and recompute the tile.  O / l is unchanged by the choice of reference, and the
// references are integers, so the bf16 probabilities do not depend on when
// the reference was raised (they differ by exact powers of two).
//
// Two other reference policies exist for comparison ("Fixed-max softmax is a
// numerical contract" weighs them): SM = kSoftmaxRunningMax is the textbook
// online softmax (row max of every tile, O and l rescaled every tile), and
// SM = kSoftmaxFixedFirst takes the reference from the first tile and never
// raises it -- one pass without the overflow check, exact until a later score
// exceeds the first tile's maximum by about 88 (natural log units), where
// exp overflows and the row's output becomes inf / NaN.
constexpr int kSoftmaxGuarded = 0, kSoftmaxRunningMax = 1, kSoftmaxFixedFirst = 2;

__device__ __forceinline__ float tile_row_max(const f32x16& s0, const f32x16& s1, float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
  return wave_max_pair(mx) * sl2;
}

template <int DB>
__device__ __forceinline__ void rescale(f32x16* o, float& l, float alpha) {
  l *= alpha;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
}

template <int DB, int SM = kSoftmaxGuarded>
__device__ __forceinline__ void softmax_tile(const f32x16& s0, const f32x16& s1, float sl2, float& m, float& l,
                                             f32x16* o, bf16x2* p2) {
  if constexpr (SM == kSoftmaxRunningMax) {
    const float mnew = fmaxf(m, tile_row_max(s0, s1, sl2));
    rescale<DB>(o, l, __builtin_amdgcn_exp2f(m - mnew));  // first tile: exp2(-inf) = 0 on zeros
    m = mnew;
    l += tile_probs(s0, s1, sl2, m, p2);
  } else if constexpr (SM == kSoftmaxFixedFirst) {
    if (m == -INFINITY) m = ceilf(tile_row_max(s0, s1, sl2));  // first tile only (every row at once)
    l += tile_probs(s0, s1, sl2, m, p2);
  } else {
    float lt = tile_probs(s0, s1, sl2, m, p2);
    if (__ballot(!(lt <= 0x1p16f))) {  // first tile (m = -inf gives inf/NaN) or a big jump
      const float mnew = fmaxf(m, ceilf(tile_row_max(s0, s1, sl2)));  // integer: later raises rescale by 2^n
      rescale<DB>(o, l, __builtin_amdgcn_exp2f(m - mnew));
      m = mnew;
      lt = tile_probs(s0, s1, sl2, m, p2);
    }
    l += lt;
  }
}

// Final normalisation and store of one wavefront's 32 x D output block: the
// lane writes its query row's DB*4 float4s (orow null: nothing stored).
// Returns lse (natural log).
template <int DB>
__device__ __forceinline__ float finish_store(const f32x16* o, float m, float l, float* __restrict__ orow,
                                              int half) {
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  if (orow) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(orow + b * 32 + rq * 8 + half * 4) =
            make_float4(o[b][rq * 4] * inv, o[b][rq * 4 + 1] * inv, o[b][rq * 4 + 2] * inv, o[b][rq * 4 + 3] * inv);
  }
  return (m + __builtin_amdgcn_logf(lt)) * kLn2;
}

}  // namespace wf
