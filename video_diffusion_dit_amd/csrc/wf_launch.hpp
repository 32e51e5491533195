// Internal host-side interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace wf {

// Per-kernel timing hooks (capi.hip): when timing is enabled, a HIP event is
// recorded on the launch stream before and after the launch.
int prof_begin(const char* name, hipStream_t s);
void prof_end(int slot, hipStream_t s);

template <class F>
hipError_t wf_launch(const char* name, hipStream_t s, F&& launch) {
  const int slot = prof_begin(name, s);
  launch();
  const hipError_t e = hipGetLastError();
  prof_end(slot, s);
  return e;
}

// 3D RoPE of Q and K (bf16 [B][Hh][T*H*W][D], D = 64 or 128), precision 32 or 64; out may equal in.
hipError_t launch_rope_qk(const void* q, const void* k, void* qo, void* ko, int B, int Hh, int T, int H,
                          int W, int D, double theta, int precision, hipStream_t s);

// Dense attention.
size_t dense_workspace_bytes(int BH, int N, int D);
// softmax_mode: 0 guarded integer reference, 1 running max, 2 fixed first-tile reference.
hipError_t launch_dense(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                        int N, int D, float scale, int softmax_mode, void* ws, hipStream_t s);
// The same with the library's static per-GPU scratch (noalloc.hip) as the workspace; the caller
// has checked dense_workspace_bytes() against its size.
hipError_t launch_dense_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                                int N, int D, float scale, hipStream_t s);

// VSA workspace layout (byte offsets, each 256-byte aligned).
struct VsaLayout {
  int C;
  size_t qc, kc, vct, qbar, kbar, vbt, scores, stat, ocoarse, flag, total;
};
VsaLayout vsa_layout(int BH, int T, int H, int W, int D);
// rope_theta > 0: Q and K pass through the 3D RoPE with that frequency base in the gather,
// rotated in fp32 or fp64 (rope_precision 32 or 64).
hipError_t launch_vsa_coarse(const void* q, const void* k, const void* v, int BH, int T, int H,
                             int W, int D, float scale, int topk, double rope_theta,
                             int rope_precision, int* idx, float* scores_out, void* ws, hipStream_t s);
hipError_t launch_vsa_check(const int* idx, int BH, int C, int topk, void* ws, size_t flag_off,
                            hipStream_t s, int* bad);
hipError_t launch_vsa_fine(const void* ws, const int* idx, int BH, int T, int H, int W, int D,
                           float scale, int topk, int softmax_mode, float* o, float* lse, hipStream_t s);
hipError_t launch_vsa_fine_gated(void* ws, const int* idx, const void* gate, int BH, int T, int H,
                                 int W, int D, float scale, int topk, float* o, float* lse,
                                 float* o_coarse, hipStream_t s);
// VSA in one call (coarse stage and fine stage; no cube-ordered copies of Q and K); with a gate,
// the coarse-branch output (into o_coarse when not null) and the gated merge.
hipError_t launch_vsa_onecall(const void* q, const void* k, const void* v, int BH, int T, int H, int W, int D,
                              float scale, int topk, int* idx, const void* gate, float* o, float* lse,
                              float* o_coarse, void* ws, hipStream_t s);

// Sliding-tile attention: 6x8x8-token tiles, a (wt, wh, ww)-tile window per query tile; the
// gather into 1x8x8 slabs, the slab plan (and the tile plan into plan_out, int32
// [tiles][wt*wh*ww], when not null), the fine stage.  Grids must be whole tiles.
struct StaLayout {
  size_t qc, kc, vct, plan, total;
};
StaLayout sta_layout(int BH, int T, int H, int W, int D, int k);
int sta_slabs(int T, int H, int W);
hipError_t launch_sta(const void* q, const void* k, const void* v, int BH, int T, int H, int W, int D,
                      float scale, int wt, int wh, int ww, float* o, float* lse, int* plan_out, void* ws,
                      hipStream_t s);

}  // namespace wf
