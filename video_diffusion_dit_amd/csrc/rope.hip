// Standalone 3D RoPE of Q and K (the form dense attention uses; VSA fuses the
// same rotation into its gather).  Definition and precision: wf_rope.hpp.
#include "wf_device.hpp"
#include "wf_launch.hpp"
#include "wf_rope.hpp"

namespace wf {

constexpr int kRopeTokens = 64;  // tokens of one grid row (fixed b, t, h) per workgroup
constexpr int kRopeHeads = 8;    // heads per workgroup (the table is shared by all of them)

// One workgroup per (b, t, h, block of up to 64 w, group of up to 8 heads).
// Table in LDS: the t part's and the h part's (cos, sin) for this row, then
// the w part's for each of the block's w.  Then every 16-byte chunk of the
// block's Q and K rows is rotated and written (in place when out == in); a
// thread loads all of its chunks of a head's row block before rotating any.
template <int D, int P>
__global__ void __launch_bounds__(256) wf_rope_qk_kernel(
    const uint16_t* q, const uint16_t* k, uint16_t* qo, uint16_t* ko, int Hh, int T, int H, int W,
    int wblocks, int hgroups, double theta) {
  using CS = RopeCS<P>;
  constexpr RopeSplit sp = rope_split(D);
  constexpr int NTAB = sp.t2 + sp.h2 + sp.w2 * kRopeTokens, CPR = D / 8;  // CPR: 16-byte chunks per row
  constexpr int RSTEP = 256 / CPR, NI = kRopeTokens / RSTEP;  // token rows per pass; passes
  __shared__ CS tab[NTAB];
  int item = blockIdx.x;
  const int hg = item % hgroups;
  item /= hgroups;
  const int wb = item % wblocks;
  item /= wblocks;
  const int h = item % H;
  item /= H;
  const int t = item % T, b = item / T;
  const int w0 = wb * kRopeTokens, nw = min(kRopeTokens, W - w0);
  for (int e = threadIdx.x; e < NTAB; e += blockDim.x) {
    if (e < sp.t2)
      tab[e] = rope_cs<CS>(t, rope_freq(e, 2 * sp.t2, theta));
    else if (e < sp.t2 + sp.h2)
      tab[e] = rope_cs<CS>(h, rope_freq(e - sp.t2, 2 * sp.h2, theta));
    else {
      const int i = (e - sp.t2 - sp.h2) / kRopeTokens, wl = (e - sp.t2 - sp.h2) % kRopeTokens;
      tab[e] = rope_cs<CS>(w0 + wl, rope_freq(i, 2 * sp.w2, theta));
    }
  }
  __syncthreads();
  const long N = (long)T * H * W;
  const long tok0 = ((long)t * H + h) * W + w0;
  const int h_end = min(Hh, (hg + 1) * kRopeHeads);
  const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  for (int hh = hg * kRopeHeads; hh < h_end; ++hh) {
    const long base = (((long)b * Hh + hh) * N + tok0) * D + c * 8;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint16_t* src = which ? k : q;
      uint16_t* dst = which ? ko : qo;
      uint4 u[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int wl = r0 + i * RSTEP;
        u[i] = wl < nw ? *reinterpret_cast<const uint4*>(src + base + (long)wl * D) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int wl = r0 + i * RSTEP;
        if (wl < nw)
          *reinterpret_cast<uint4*>(dst + base + (long)wl * D) = rope_rotate_chunk(u[i], c * 4, [&](int p) {
            return p < sp.t2 + sp.h2 ? tab[p] : tab[sp.t2 + sp.h2 + (p - sp.t2 - sp.h2) * kRopeTokens + wl];
          });
      }
    }
  }
}

hipError_t launch_rope_qk(const void* q, const void* k, void* qo, void* ko, int B, int Hh, int T, int H,
                          int W, int D, double theta, int precision, hipStream_t s) {
  const int wblocks = (W + kRopeTokens - 1) / kRopeTokens, hgroups = (Hh + kRopeHeads - 1) / kRopeHeads;
  const dim3 grid((unsigned)((long)B * T * H * wblocks * hgroups));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<uint16_t*>(qo), static_cast<uint16_t*>(ko), Hh, T, H, W, wblocks, hgroups, theta);
  };
  return wf_launch(precision == 64 ? "wf_rope_qk_fp64" : "wf_rope_qk", s, [&] {
    if (D == 128)
      precision == 64 ? go(wf_rope_qk_kernel<128, 64>) : go(wf_rope_qk_kernel<128, 32>);
    else
      precision == 64 ? go(wf_rope_qk_kernel<64, 64>) : go(wf_rope_qk_kernel<64, 32>);
  });
}

}  // namespace wf
