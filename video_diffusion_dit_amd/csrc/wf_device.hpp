// Device-side building blocks shared by the dense and VSA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
// The running maximum used as the softmax reference is only raised when a new
// score exceeds it by more than this many powers of two; until then the
// probabilities stay below 2^kLazy (safe in bf16 and fp32) and the O / l
// accumulators need no rescaling.  O and l share the reference, so the final
// O / l is unchanged (an exact identity, not an approximation).
constexpr float kLazy = 8.f;
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

// Key order used for V^T tiles inside every group of 16 keys: keys 4..7 and
// 8..11 trade places (bits 2 and 3 of the index swap; an involution).  It is
// the order in which a 32x32 MFMA result holds its rows in one lane pair, so
// the probabilities feed the PV product straight from the score registers.
__host__ __device__ constexpr int perm16(int n) {
  return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max_pair(float x) {  // max over lanes L and L^32
  return fmaxf(x, __shfl_xor(x, 32));
}

// One wavefront owns 32 query rows; a workgroup of NW wavefronts shares K and
// V^T tiles of BN = 64 keys staged through LDS (double buffered, register
// prefetch of the next tile while the current one is consumed).
//
// Per wavefront and tile, with lane L (j = L % 32, half = L / 32):
//   S^T (64 x 32) = K_tile (64 x D) . Q^T (D x 32)   two 32x32 blocks, MFMA 32x32x16 bf16
//     - A operand: K rows from LDS, B operand: Q held in registers;
//     - lane L ends up holding query j and key rows 8*(r/4) + 4*half + r%4 of
//       each block, so the row max / sum of query j needs only lanes L, L^32.
//   online softmax in the exp2 domain: m (running max, log2 units), l (sum of
//     the bf16-rounded probabilities, per lane, merged at the end);
//   O^T (D x 32) += V^T_tile (D x 64) . P^T (64 x 32)  D/32 blocks x 4 k-steps
//     - A operand: V^T rows from LDS (keys stored in perm16 order),
//       B operand: P^T straight from the score registers.
template <int D, int NW>
struct Tile {
  static constexpr int BN = 64;
  static constexpr int NT = NW * 64;
  static constexpr int KSTR = D + 8;          // LDS row stride (elements) of the K tile
  static constexpr int VSTR = BN + 8;         // LDS row stride of the V^T tile
  static constexpr int KELEMS = BN * KSTR;
  static constexpr int VELEMS = D * VSTR;
  static constexpr int STAGE = KELEMS + VELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int KCH = BN * D / 8 / NT;  // 16-byte chunks per thread, K tile
  static constexpr int VCH = D * BN / 8 / NT;  // same, V^T tile
  static constexpr int KROWCH = D / 8;         // chunks per K row
  static constexpr int VROWCH = BN / 8;        // chunks per V^T row
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");

  uint4 kreg[KCH];
  uint4 vreg[VCH];

  // Global -> registers.  kg: row-major [BN][D] (rows >= krows read as zero);
  // vg: V^T rows of BN keys, row d at vg + d * vld.
  __device__ __forceinline__ void fetch(const uint16_t* __restrict__ kg, int krows,
                                        const uint16_t* __restrict__ vg, long vld, int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = i * NT + tid;
      const int r = id / KROWCH, c = id % KROWCH;
      kreg[i] = (r < krows) ? *reinterpret_cast<const uint4*>(kg + (long)r * D + c * 8)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int id = i * NT + tid;
      const int d = id / VROWCH, c = id % VROWCH;
      vreg[i] = *reinterpret_cast<const uint4*>(vg + (long)d * vld + c * 8);
    }
  }

  // Registers -> LDS stage.
  __device__ __forceinline__ void stash(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = i * NT + tid;
      const int r = id / KROWCH, c = id % KROWCH;
      *reinterpret_cast<uint4*>(lds + r * KSTR + c * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int id = i * NT + tid;
      const int d = id / VROWCH, c = id % VROWCH;
      *reinterpret_cast<uint4*>(lds + KELEMS + d * VSTR + c * 8) = vreg[i];
    }
  }
};

__device__ __forceinline__ void wait_tile_copies() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's global->LDS copies landed
}

struct P4 {
  bf16x2 v[4];
};

// Per-wavefront attention state for 32 query rows.
template <int D>
struct RowState {
  static constexpr int KK = D / 16;  // k-steps of the QK^T product
  static constexpr int DB = D / 32;  // 32-row blocks of O^T
  bf16x8 qop[KK];
  f32x16 o[DB];
  float m;  // running max of scale*log2(e)*s (log2 units)
  float l;  // this lane's share of the running sum

  // q_row: this lane's query row (D bf16) or nullptr for a zero row.
  __device__ __forceinline__ void init(const uint16_t* __restrict__ q_row, int half) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 u = q_row ? *reinterpret_cast<const uint4*>(q_row + kk * 16 + half * 8)
                      : make_uint4(0, 0, 0, 0);
      qop[kk] = as_bf16x8(u);
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
    m = -INFINITY;
    l = 0.f;
  }

  // S^T for the 64 keys of the LDS stage.
  __device__ __forceinline__ void scores(const uint16_t* lds, int j, int half, f32x16& s0,
                                         f32x16& s1) const {
    using T = Tile<D, 1>;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + j * T::KSTR + kk * 16 + half * 8));
      const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4*>(lds + (32 + j) * T::KSTR + kk * 16 + half * 8));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qop[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qop[kk], s1, 0, 0, 0);
    }
  }

  // Online softmax update with scores s0/s1 (masked entries already -inf),
  // then O^T += V^T P^T from the LDS stage.
  __device__ __forceinline__ void update(const uint16_t* lds, int j, int half, const f32x16& s0,
                                         const f32x16& s1, float sl2) {
    using T = Tile<D, 1>;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);  // v_max3 chain
    mx = wave_max_pair(mx) * sl2;
    if (__ballot(mx > m + kLazy)) {  // wave-uniform: raise the reference, rescale O and l
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
    }
    const float nm = -m;
    bf16x2 p2[16];  // probabilities, two per register, in score-register order
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
    float la = 0.f, lb = 0.f;  // row sum of the bf16 probabilities (what the MFMA consumes)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      la = __builtin_amdgcn_fdot2_f32_bf16(p2[i], one2, la, false);
      lb = __builtin_amdgcn_fdot2_f32_bf16(p2[i + 1], one2, lb, false);
    }
    l += la + lb;
    const uint16_t* vt = lds + T::KELEMS;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int base = (ks / 2) * 8 + (ks % 2) * 4;
      const bf16x8 p = __builtin_bit_cast(bf16x8, P4{p2[base], p2[base + 1], p2[base + 2], p2[base + 3]});
#pragma unroll
      for (int b = 0; b < DB; ++b)
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(vt + (b * 32 + j) * T::VSTR + ks * 16 + half * 8)),
            p, o[b], 0, 0, 0);
    }
  }

  // Final normalisation.  Returns this query's lse (natural log); scales o by 1/l.
  __device__ __forceinline__ float finish() {
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[b][r] *= inv;
    return (m + __builtin_amdgcn_logf(lt)) * kLn2;
  }

  // Store the 32 x D block: this lane writes its query row's 4*DB float4s.
  __device__ __forceinline__ void store(float* __restrict__ o_row, int half) const {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(o_row + b * 32 + rq * 8 + half * 4) =
            make_float4(o[b][rq * 4 + 0], o[b][rq * 4 + 1], o[b][rq * 4 + 2], o[b][rq * 4 + 3]);
  }
};

// Key row (0..63 inside the stage) held by register r of block kb in lane half `half`.
__device__ __forceinline__ int key_row(int kb, int r, int half) {
  return kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
}

}  // namespace wf
