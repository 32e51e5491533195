// C ABI of libwfattn.so: argument validation, status codes, dispatch, and the
// optional per-kernel event timing.  Declarations and contracts: wf_attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "wf_attn.h"
#include "wf_launch.hpp"

namespace {

thread_local std::string g_detail;

int32_t fail(wf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(wf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

int32_t ok() {
  g_detail.clear();
  return WF_OK;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(WF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define WF_CHECK_PTR(p)                                                      \
  do {                                                                       \
    if (!(p)) return fail(WF_ERR_INVALID_ARG, "%s is NULL", #p);             \
    if (!aligned16(p)) return fail(WF_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

#define WF_CHECK_OPT_PTR(p)                                                  \
  do {                                                                       \
    if ((p) && !aligned16(p)) return fail(WF_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

// Largest element count of one [B][Hh][N][D] tensor the kernels index with
// 64-bit offsets but 32-bit per-head offsets: N * D must fit in int32.
bool sizes_ok(long long B, long long Hh, long long N, long long D) {
  if (B < 1 || Hh < 1 || N < 1 || D < 1) return false;
  if (N * D >= (1ll << 31)) return false;
  if (B * Hh >= (1ll << 24)) return false;
  return true;
}

// -------------------------------------------------------------- timing state
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
size_t g_pool_used = 0;
long long g_dropped = 0;
constexpr size_t kMaxRecs = 65536;

hipEvent_t pool_event() {
  if (g_pool_used < g_pool.size()) return g_pool[g_pool_used++];
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  g_pool.push_back(e);
  ++g_pool_used;
  return e;
}

}  // namespace

namespace wf {

int prof_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return -1;
  if (g_recs.size() >= kMaxRecs) {
    ++g_dropped;
    return -1;
  }
  hipEvent_t a = pool_event(), b = pool_event();
  if (!a || !b) return -1;
  (void)hipEventRecord(a, s);
  g_recs.push_back({name, a, b});
  return (int)g_recs.size() - 1;
}

void prof_end(int slot, hipStream_t s) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot < (int)g_recs.size()) (void)hipEventRecord(g_recs[slot].b, s);
}

}  // namespace wf

extern "C" {

const char* wf_status_string(int32_t status) {
  switch (status) {
    case WF_OK: return "WF_OK";
    case WF_ERR_INVALID_ARG: return "WF_ERR_INVALID_ARG";
    case WF_ERR_UNSUPPORTED: return "WF_ERR_UNSUPPORTED";
    case WF_ERR_WORKSPACE: return "WF_ERR_WORKSPACE";
    case WF_ERR_BAD_INDEX: return "WF_ERR_BAD_INDEX";
    case WF_ERR_HIP: return "WF_ERR_HIP";
    default: return "WF_UNKNOWN_STATUS";
  }
}

const char* wf_last_error_detail(void) { return g_detail.c_str(); }

int32_t wf_abi_version(void) { return 4; }

size_t wf_attn_dense_workspace_bytes(int32_t B, int32_t Hh, int32_t N, int32_t D) {
  if (!sizes_ok(B, Hh, N, D)) return 0;
  return wf::dense_workspace_bytes(B * Hh, N, D);
}

// Argument checks shared by the dense entry points (everything but the workspace).
static int32_t dense_checks(const void* q, const void* k, const void* v, float* o, float* lse, int32_t B,
                            int32_t Hh, int32_t N, int32_t D, float scale) {
  WF_CHECK_PTR(q);
  WF_CHECK_PTR(k);
  WF_CHECK_PTR(v);
  WF_CHECK_PTR(o);
  WF_CHECK_OPT_PTR(lse);
  if (!sizes_ok(B, Hh, N, D))
    return fail(WF_ERR_INVALID_ARG, "bad sizes B=%d Hh=%d N=%d D=%d", B, Hh, N, D);
  if (D != 64 && D != 128) return fail(WF_ERR_UNSUPPORTED, "head dimension %d (64 or 128)", D);
  if ((long long)B * Hh * ((N + 63) / 64) >= (1ll << 31))  // the V^T transpose's grid, the largest
    return fail(WF_ERR_UNSUPPORTED, "B=%d Hh=%d N=%d: too many workgroups for one launch", B, Hh, N);
  // one head's K and V^T are read through buffer descriptors with 32-bit byte counts and offsets
  if ((long long)((N + 63) / 64) * 64 * D * 2 >= (1ll << 31))
    return fail(WF_ERR_UNSUPPORTED, "N=%d D=%d: one head's K and V^T must stay below 2 GiB", N, D);
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(WF_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)scale);
  return WF_OK;
}

static int32_t dense(const void* q, const void* k, const void* v, float* o, float* lse, int32_t B,
                     int32_t Hh, int32_t N, int32_t D, float scale, int32_t softmax_mode,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t st = dense_checks(q, k, v, o, lse, B, Hh, N, D, scale)) return st;
  const size_t need = wf::dense_workspace_bytes(B * Hh, N, D);
  if (!workspace || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  WF_CHECK_PTR(workspace);
  hipError_t e = wf::launch_dense(q, k, v, o, lse, B * Hh, N, D, scale, softmax_mode, workspace,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense launch");
  return ok();
}

int32_t wf_attn_dense(const void* q, const void* k, const void* v, float* o, float* lse, int32_t B,
                      int32_t Hh, int32_t N, int32_t D, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return dense(q, k, v, o, lse, B, Hh, N, D, scale, WF_SOFTMAX_GUARDED, workspace, workspace_bytes,
               stream);
}

int32_t wf_attn_dense_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int32_t B,
                              int32_t Hh, int32_t N, int32_t D, float scale, void* stream) {
  if (int32_t st = dense_checks(q, k, v, o, lse, B, Hh, N, D, scale)) return st;
  const size_t need = wf::dense_workspace_bytes(B * Hh, N, D);
  if (need > (size_t)WF_DENSE_NOALLOC_SCRATCH_BYTES)
    return fail(WF_ERR_WORKSPACE, "B=%d Hh=%d N=%d D=%d needs %zu bytes of scratch; the static scratch holds %zu",
                B, Hh, N, D, need, (size_t)WF_DENSE_NOALLOC_SCRATCH_BYTES);
  hipError_t e = wf::launch_dense_noalloc(q, k, v, o, lse, B * Hh, N, D, scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense (static scratch) launch");
  return ok();
}

static bool softmax_mode_ok(int32_t mode) {
  return mode == WF_SOFTMAX_GUARDED || mode == WF_SOFTMAX_RUNNING_MAX || mode == WF_SOFTMAX_FIXED_FIRST_TILE;
}

int32_t wf_attn_dense_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                         int32_t B, int32_t Hh, int32_t N, int32_t D, float scale,
                         int32_t softmax_mode, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!softmax_mode_ok(softmax_mode)) return fail(WF_ERR_INVALID_ARG, "softmax_mode %d", softmax_mode);
  return dense(q, k, v, o, lse, B, Hh, N, D, scale, softmax_mode, workspace, workspace_bytes, stream);
}

int32_t wf_vsa_num_cubes(int32_t T, int32_t H, int32_t W) {
  if (T < 1 || H < 1 || W < 1) return 0;
  const long long C = (long long)((T + 3) / 4) * ((H + 3) / 4) * ((W + 3) / 4);
  return C > (1 << 20) ? 0 : (int32_t)C;
}

static int32_t vsa_check_sizes(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D) {
  if (T < 1 || H < 1 || W < 1)
    return fail(WF_ERR_INVALID_ARG, "bad grid T=%d H=%d W=%d", T, H, W);
  const int32_t C = wf_vsa_num_cubes(T, H, W);
  if (C == 0) return fail(WF_ERR_INVALID_ARG, "grid %dx%dx%d too large", T, H, W);
  const long long Np = (long long)C * 64;
  if (!sizes_ok(B, Hh, Np, D))
    return fail(WF_ERR_INVALID_ARG, "bad sizes B=%d Hh=%d padded tokens=%lld D=%d", B, Hh, Np, D);
  if (D != 128) return fail(WF_ERR_UNSUPPORTED, "VSA head dimension %d (only 128)", D);
  if (C > 4096) return fail(WF_ERR_UNSUPPORTED, "%d cubes (at most 4096)", C);
  if ((long long)B * Hh * C >= (1ll << 31))  // one workgroup per (head, cube) in the gather and fine stage
    return fail(WF_ERR_UNSUPPORTED, "B=%d Hh=%d with %d cubes: too many workgroups for one launch", B, Hh, C);
  if ((long long)C * C >= (1ll << 31))
    return fail(WF_ERR_UNSUPPORTED, "%d cubes: score matrix too large", C);
  return WF_OK;
}

size_t wf_vsa_workspace_bytes(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D) {
  if (vsa_check_sizes(B, Hh, T, H, W, D) != WF_OK) return 0;
  return wf::vsa_layout(B * Hh, T, H, W, D).total;
}

static int32_t vsa_coarse(const void* q, const void* k, const void* v, int32_t B, int32_t Hh,
                          int32_t T, int32_t H, int32_t W, int32_t D, float scale, int32_t topk,
                          double rope_theta, int32_t rope_precision, int32_t* idx,
                          float* coarse_scores, void* workspace, size_t workspace_bytes,
                          void* stream) {
  WF_CHECK_PTR(q);
  WF_CHECK_PTR(k);
  WF_CHECK_PTR(v);
  WF_CHECK_PTR(idx);
  WF_CHECK_OPT_PTR(coarse_scores);
  if (int32_t st = vsa_check_sizes(B, Hh, T, H, W, D)) return st;
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(WF_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)scale);
  const int32_t C = wf_vsa_num_cubes(T, H, W);
  if (topk < 1 || topk > C) return fail(WF_ERR_INVALID_ARG, "topk %d outside [1, %d]", topk, C);
  const size_t need = wf::vsa_layout(B * Hh, T, H, W, D).total;
  if (!workspace || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  WF_CHECK_PTR(workspace);
  hipError_t e = wf::launch_vsa_coarse(q, k, v, B * Hh, T, H, W, D, scale, topk, rope_theta,
                                       rope_precision, idx, coarse_scores, workspace,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "VSA coarse launch");
  return ok();
}

int32_t wf_vsa_coarse_topk(const void* q, const void* k, const void* v, int32_t B, int32_t Hh,
                           int32_t T, int32_t H, int32_t W, int32_t D, float scale, int32_t topk,
                           int32_t* idx, float* coarse_scores, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return vsa_coarse(q, k, v, B, Hh, T, H, W, D, scale, topk, 0.0, 0, idx, coarse_scores, workspace,
                    workspace_bytes, stream);
}

int32_t wf_vsa(const void* q, const void* k, const void* v, int32_t B, int32_t Hh, int32_t T, int32_t H,
               int32_t W, int32_t D, float scale, int32_t topk, int32_t* idx, const void* gate, float* o,
               float* lse, float* o_coarse, void* workspace, size_t workspace_bytes, void* stream) {
  WF_CHECK_PTR(q);
  WF_CHECK_PTR(k);
  WF_CHECK_PTR(v);
  WF_CHECK_PTR(idx);
  WF_CHECK_OPT_PTR(gate);
  WF_CHECK_PTR(o);
  WF_CHECK_OPT_PTR(lse);
  WF_CHECK_OPT_PTR(o_coarse);
  if (o_coarse && !gate) return fail(WF_ERR_INVALID_ARG, "o_coarse given without a gate");
  if (int32_t st = vsa_check_sizes(B, Hh, T, H, W, D)) return st;
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(WF_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)scale);
  const int32_t C = wf_vsa_num_cubes(T, H, W);
  if (topk < 1 || topk > C) return fail(WF_ERR_INVALID_ARG, "topk %d outside [1, %d]", topk, C);
  const size_t need = wf::vsa_layout(B * Hh, T, H, W, D).total;
  if (!workspace || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  WF_CHECK_PTR(workspace);
  hipError_t e = wf::launch_vsa_onecall(q, k, v, B * Hh, T, H, W, D, scale, topk, idx, gate, o, lse, o_coarse,
                                        workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "VSA launch");
  return ok();
}

int32_t wf_vsa_coarse_topk_rope(const void* q, const void* k, const void* v, int32_t B, int32_t Hh,
                                int32_t T, int32_t H, int32_t W, int32_t D, float scale,
                                int32_t topk, double rope_theta, int32_t rope_precision,
                                int32_t* idx, float* coarse_scores, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!isfinite(rope_theta) || !(rope_theta > 0.0))
    return fail(WF_ERR_INVALID_ARG, "rope_theta %g must be finite and > 0", rope_theta);
  if (rope_precision != 32 && rope_precision != 64)
    return fail(WF_ERR_INVALID_ARG, "rope_precision %d (32 or 64)", rope_precision);
  return vsa_coarse(q, k, v, B, Hh, T, H, W, D, scale, topk, rope_theta, rope_precision, idx,
                    coarse_scores, workspace, workspace_bytes, stream);
}

int32_t wf_rope_qk(const void* q, const void* k, void* q_out, void* k_out, int32_t B, int32_t Hh,
                   int32_t T, int32_t H, int32_t W, int32_t D, double theta, int32_t precision,
                   void* stream) {
  WF_CHECK_PTR(q);
  WF_CHECK_PTR(k);
  WF_CHECK_PTR(q_out);
  WF_CHECK_PTR(k_out);
  if (T < 1 || H < 1 || W < 1) return fail(WF_ERR_INVALID_ARG, "bad grid T=%d H=%d W=%d", T, H, W);
  const long long N = (long long)T * H * W;
  if (!sizes_ok(B, Hh, N, D))
    return fail(WF_ERR_INVALID_ARG, "bad sizes B=%d Hh=%d N=%lld D=%d", B, Hh, N, D);
  if (D != 64 && D != 128) return fail(WF_ERR_UNSUPPORTED, "RoPE head dimension %d (64 or 128)", D);
  if ((long long)B * T * H * ((W + 63) / 64) * ((Hh + 7) / 8) >= (1ll << 31))
    return fail(WF_ERR_UNSUPPORTED, "grid %dx%dx%d with B=%d Hh=%d: too many workgroups", T, H, W, B, Hh);
  if (!isfinite(theta) || !(theta > 0.0))
    return fail(WF_ERR_INVALID_ARG, "theta %g must be finite and > 0", theta);
  if (precision != 32 && precision != 64)
    return fail(WF_ERR_INVALID_ARG, "precision %d (32 or 64)", precision);
  hipError_t e = wf::launch_rope_qk(q, k, q_out, k_out, B, Hh, T, H, W, D, theta, precision,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "RoPE launch");
  return ok();
}

// Checks shared by the fine-stage entry points, then the opt-in plan check.
static int32_t vsa_fine_checks(const void* workspace, size_t workspace_bytes, const int32_t* idx,
                               int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                               float scale, int32_t topk, float* o, float* lse, hipStream_t s) {
  WF_CHECK_PTR(idx);
  WF_CHECK_PTR(o);
  WF_CHECK_OPT_PTR(lse);
  if (int32_t st = vsa_check_sizes(B, Hh, T, H, W, D)) return st;
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(WF_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)scale);
  const int32_t C = wf_vsa_num_cubes(T, H, W);
  if (topk < 1 || topk > C) return fail(WF_ERR_INVALID_ARG, "topk %d outside [1, %d]", topk, C);
  const wf::VsaLayout L = wf::vsa_layout(B * Hh, T, H, W, D);
  if (!workspace || workspace_bytes < L.total)
    return fail(WF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                L.total);
  WF_CHECK_PTR(workspace);
  const char* val = getenv("WF_VALIDATE");
  if (val && val[0] == '1') {
    int bad = 0;
    hipError_t e = wf::launch_vsa_check(idx, B * Hh, C, topk, const_cast<void*>(workspace), L.flag,
                                        s, &bad);
    if (e != hipSuccess) return hip_fail(e, "VSA plan check");
    if (bad) return fail(WF_ERR_BAD_INDEX, "top-k plan has an index outside [0, %d) or a row that is not strictly ascending", C);
  }
  return WF_OK;
}

int32_t wf_vsa_fine(const void* workspace, size_t workspace_bytes, const int32_t* idx, int32_t B,
                    int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D, float scale,
                    int32_t topk, float* o, float* lse, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int32_t st = vsa_fine_checks(workspace, workspace_bytes, idx, B, Hh, T, H, W, D, scale, topk,
                                   o, lse, s))
    return st;
  hipError_t e = wf::launch_vsa_fine(workspace, idx, B * Hh, T, H, W, D, scale, topk,
                                     WF_SOFTMAX_GUARDED, o, lse, s);
  if (e != hipSuccess) return hip_fail(e, "VSA fine launch");
  return ok();
}

int32_t wf_vsa_fine_ex(const void* workspace, size_t workspace_bytes, const int32_t* idx,
                       int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                       float scale, int32_t topk, int32_t softmax_mode, float* o, float* lse,
                       void* stream) {
  if (!softmax_mode_ok(softmax_mode)) return fail(WF_ERR_INVALID_ARG, "softmax_mode %d", softmax_mode);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int32_t st = vsa_fine_checks(workspace, workspace_bytes, idx, B, Hh, T, H, W, D, scale, topk,
                                   o, lse, s))
    return st;
  hipError_t e = wf::launch_vsa_fine(workspace, idx, B * Hh, T, H, W, D, scale, topk, softmax_mode,
                                     o, lse, s);
  if (e != hipSuccess) return hip_fail(e, "VSA fine launch");
  return ok();
}

int32_t wf_vsa_fine_gated(void* workspace, size_t workspace_bytes, const int32_t* idx,
                          const void* gate, int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W,
                          int32_t D, float scale, int32_t topk, float* o, float* lse,
                          float* o_coarse, void* stream) {
  WF_CHECK_PTR(gate);
  WF_CHECK_OPT_PTR(o_coarse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int32_t st = vsa_fine_checks(workspace, workspace_bytes, idx, B, Hh, T, H, W, D, scale, topk,
                                   o, lse, s))
    return st;
  hipError_t e = wf::launch_vsa_fine_gated(workspace, idx, gate, B * Hh, T, H, W, D, scale, topk, o,
                                           lse, o_coarse, s);
  if (e != hipSuccess) return hip_fail(e, "VSA gated fine launch");
  return ok();
}

// Sliding-tile attention runs on the two token grids it is tuned for and refuses every other
// grid before any GPU work ("推理优化", approximate attention, entry "sta").  Both are whole
// numbers of 6x8x8 tiles.
static bool sta_tuned_grid(int32_t T, int32_t H, int32_t W) {
  return (T == 36 && H == 48 && W == 48) || (T == 18 && H == 48 && W == 80);
}

static int32_t sta_check(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D, int32_t wt,
                         int32_t wh, int32_t ww) {
  if (!sta_tuned_grid(T, H, W))
    return fail(WF_ERR_UNSUPPORTED, "sliding-tile attention runs on the tuned grids 36x48x48 and 18x48x80 only, "
                "not %dx%dx%d", T, H, W);
  if (int32_t st = vsa_check_sizes(B, Hh, T, H, W, D)) return st;
  const int nt = T / 6, nh = H / 8, nw = W / 8;
  if (wt < 1 || wt > nt || wh < 1 || wh > nh || ww < 1 || ww > nw)
    return fail(WF_ERR_INVALID_ARG, "window %dx%dx%d tiles must fit the tile grid %dx%dx%d", wt, wh, ww, nt, nh,
                nw);
  if ((long long)B * Hh * wf::sta_slabs(T, H, W) >= (1ll << 31))
    return fail(WF_ERR_UNSUPPORTED, "B=%d Hh=%d: too many workgroups for one launch", B, Hh);
  return WF_OK;
}

size_t wf_sta_workspace_bytes(int32_t B, int32_t Hh, int32_t T, int32_t H, int32_t W, int32_t D,
                              int32_t wt, int32_t wh, int32_t ww) {
  if (sta_check(B, Hh, T, H, W, D, wt, wh, ww) != WF_OK) return 0;
  return wf::sta_layout(B * Hh, T, H, W, D, wt * wh * ww).total;
}

int32_t wf_sta(const void* q, const void* k, const void* v, int32_t B, int32_t Hh, int32_t T, int32_t H,
               int32_t W, int32_t D, float scale, int32_t wt, int32_t wh, int32_t ww, float* o, float* lse,
               int32_t* plan, void* workspace, size_t workspace_bytes, void* stream) {
  WF_CHECK_PTR(q);
  WF_CHECK_PTR(k);
  WF_CHECK_PTR(v);
  WF_CHECK_PTR(o);
  WF_CHECK_OPT_PTR(lse);
  WF_CHECK_OPT_PTR(plan);
  if (int32_t st = sta_check(B, Hh, T, H, W, D, wt, wh, ww)) return st;
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(WF_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)scale);
  const size_t need = wf::sta_layout(B * Hh, T, H, W, D, wt * wh * ww).total;
  if (!workspace || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0, need);
  WF_CHECK_PTR(workspace);
  hipError_t e = wf::launch_sta(q, k, v, B * Hh, T, H, W, D, scale, wt, wh, ww, o, lse, plan, workspace,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "STA launch");
  return ok();
}

int32_t wf_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (on) {
    g_recs.clear();
    g_pool_used = 0;
    g_dropped = 0;
  }
  g_on = on != 0;
  return ok();
}

int32_t wf_profile_query(const char* name, int64_t* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return fail(WF_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t n = 0;
  double tot = 0.0;
  for (const Rec& r : g_recs) {
    if (strcmp(r.name, name) != 0) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  if (n == 0) return fail(WF_ERR_INVALID_ARG, "no recorded launch of %s", name);
  *launches = n;
  *total_ms = tot;
  return ok();
}

}  // extern "C"
