// 3D rotary position embedding of Q and K on the video token grid (gfx950).
//
// Operation: "推理优化" (Inference optimization, WorldFoundry docs), section
// "Exact or numerically equivalent Wan kernels", entry fused_rope: a fused 3D
// RoPE for the Wan DiT whose rotation runs in fp32 or fp64.  The page gives no
// frequencies, so the library takes the common Wan-style definition:
//   - the head dimension D is cut into consecutive parts of
//     D - 4*floor(D/6), 2*floor(D/6) and 2*floor(D/6) dims for t, h and w;
//   - in a part of d_a dims, elements (2i, 2i+1) are pair i, rotated by
//     pos * theta^(-2i/d_a), pos being the token's 0-based coordinate on
//     that axis;
//   - (x0, x1) -> (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi), rounded
//     once to bf16 (nearest, ties to even), with the page's two precisions:
//     fp64 arithmetic throughout, or cos and sin rounded to fp32 and each
//     product and sum rounded to fp32 (no fused multiply-add, so the result
//     is one exact IEEE value that any fp32 implementation reproduces).
// The angles of a part depend on one coordinate only, so a workgroup needs
// far fewer sines and cosines than it rotates pairs: it tabulates them in LDS
// first (one fp64 sincos per table entry, rounded to fp32 for the fp32 path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wf_device.hpp"

namespace wf {

// Pairs per axis part.
struct RopeSplit {
  int t2, h2, w2;
};
__host__ __device__ constexpr RopeSplit rope_split(int D) {
  return RopeSplit{(D - 4 * (D / 6)) / 2, D / 6, D / 6};
}

// Frequency of pair i in a part of d_a dims: theta^(-2i/d_a), in fp64.
__device__ inline double rope_freq(int i, int d_a, double theta) {
  return pow(theta, (-2.0 * i) / d_a);
}

// Table entry (cos, sin) of pos * freq: fp64, or fp64 rounded to fp32.
template <class CS>
__device__ inline CS rope_cs(int pos, double freq) {
  double s, c;
  sincos((double)pos * freq, &s, &c);
  if constexpr (sizeof(CS) == sizeof(double2))
    return make_double2(c, s);
  else
    return make_float2((float)c, (float)s);
}

// fp64 -> bf16, round to nearest even, in one rounding, on the bit pattern:
// bf16 keeps 7 of fp64's 52 fraction bits, so adding 2^44 - 1 plus the kept
// part's lowest bit to the magnitude and shifting right by 45 rounds it (a
// carry moves into the exponent, which is what rounding up to the next
// binade or to infinity needs), and the exponent is rebiased from 1023 to
// 127.  Results below the normal bf16 range (|x| < 2^-126: zero, or inputs
// that are themselves that small) become a zero of the same sign; rotated
// bf16 inputs of normal size never come near it.
__device__ inline uint32_t bf16_rne_from_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag < (uint64_t)(1023 - 126) << 52) return sign;
  const uint64_t r = mag + ((1ull << 44) - 1) + ((mag >> 45) & 1);
  return sign | ((uint32_t)(r >> 45) - ((1023u - 127u) << 7));
}

// Rotate one pair packed as two bf16 (element 2i in the low half) by (c, s).
__device__ inline uint32_t rope_rotate_packed(uint32_t pair, double2 cs) {
#pragma clang fp contract(off)
  const double x0 = (double)__uint_as_float(pair << 16);
  const double x1 = (double)__uint_as_float(pair & 0xFFFF0000u);
  const double y0 = x0 * cs.x - x1 * cs.y;
  const double y1 = x0 * cs.y + x1 * cs.x;
  return bf16_rne_from_f64(y0) | (bf16_rne_from_f64(y1) << 16);
}

__device__ inline uint32_t rope_rotate_packed(uint32_t pair, float2 cs) {
#pragma clang fp contract(off)
  const float x0 = __uint_as_float(pair << 16);
  const float x1 = __uint_as_float(pair & 0xFFFF0000u);
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x0 * cs.y + x1 * cs.x;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y0, y1}, bf16x2));
}

// Table entry type of a precision (32 or 64).
template <int P>
using RopeCS = typename std::conditional<P == 64, double2, float2>::type;

// Rotate the 8 bf16 of a 16-byte chunk (pairs p0 .. p0+3); cs(p) gives a pair's (cos, sin).
template <class CS>
__device__ inline uint4 rope_rotate_chunk(uint4 u, int p0, CS&& cs) {
  u.x = rope_rotate_packed(u.x, cs(p0));
  u.y = rope_rotate_packed(u.y, cs(p0 + 1));
  u.z = rope_rotate_packed(u.z, cs(p0 + 2));
  u.w = rope_rotate_packed(u.w, cs(p0 + 3));
  return u;
}

}  // namespace wf
