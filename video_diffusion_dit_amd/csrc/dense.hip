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
  const int bh = blockIdx.y, n0 = blockIdx.x * 64, tid = threadIdx.x;
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

// One workgroup = NW wavefronts x 32 query rows of one (b, h); it sweeps all
// key tiles.  Grid: ceil(N / (32 NW)) * BH workgroups, XCD-remapped so each
// XCD walks whole heads.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 2)
wf_dense_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
             int N, int Np, int nqt, float sl2) {
  using T = Tile<D, NW>;
  __shared__ __align__(16) uint16_t lds[2 * T::STAGE];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, j = lane % 32, half = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nqt, qt = item % nqt;
  const long base = (long)bh * N;
  const uint16_t* kb = k + base * D;
  const uint16_t* vb = vt + (long)bh * D * Np;

  const int qrow = qt * 32 * NW + wave * 32 + j;
  RowState<D> st;
  st.init(qrow < N ? q + (base + qrow) * D : nullptr, half);

  T tile;
  const int ntiles = (N + 63) / 64;
  tile.fetch(kb, N, vb, Np, tid);
  tile.stash(lds, tid);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int n0 = t * 64;
    if (t + 1 < ntiles) tile.fetch(kb + (long)(n0 + 64) * D, N - n0 - 64, vb + n0 + 64, Np, tid);
    const uint16_t* cur = lds + (t & 1) * T::STAGE;
    f32x16 s0, s1;
    st.scores(cur, j, half, s0, s1);
    if (n0 + 64 > N) {  // ragged last tile: keys >= N do not exist
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (n0 + key_row(0, r, half) >= N) s0[r] = -INFINITY;
        if (n0 + key_row(1, r, half) >= N) s1[r] = -INFINITY;
      }
    }
    st.update(cur, j, half, s0, s1, sl2);
    if (t + 1 < ntiles) tile.stash(lds + ((t + 1) & 1) * T::STAGE, tid);
    __syncthreads();
  }
  const float l = st.finish();
  if (qrow < N) {
    st.store(o + (base + qrow) * D, half);
    if (lse && half == 0) lse[base + qrow] = l;
  }
}

template <int D, int NW>
static hipError_t launch_dense_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                                 float* lse, int BH, int N, float scale, uint16_t* vt,
                                 hipStream_t s) {
  const int Np = (N + 63) / 64 * 64;
  hipError_t e = wf_launch("wf_transpose_v", s, [&] {
    hipLaunchKernelGGL(wf_transpose_v<D>, dim3(Np / 64, BH), dim3(256), 0, s, v, vt, N, Np);
  });
  if (e != hipSuccess) return e;
  const int nqt = (N + 32 * NW - 1) / (32 * NW);
  const long grid = (long)nqt * BH;
  return wf_launch("wf_dense_fwd", s, [&] {
    hipLaunchKernelGGL((wf_dense_fwd<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s,
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
  if (D == 128) return launch_dense_d<128, 4>(q16, k16, v16, o, lse, BH, N, scale, vt, s);
  return launch_dense_d<64, 4>(q16, k16, v16, o, lse, BH, N, scale, vt, s);
}

}  // namespace wf
