// Dense attention with the library's own static scratch instead of a caller
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch holds V transposed per head (the same layout wf_attn_dense
// keeps in its workspace).  It is one file-scope device array per GPU, held
// from the first use on that GPU until the process ends; every call on a GPU
// shares it, so calls that overlap on one GPU (other streams, other threads)
// race on it and must be serialised by the caller.  Nothing in it has to start
// at zero: the transpose kernel writes every element the attention kernel
// reads, padding columns included, on every call.
#include <mutex>

#include "wf_attn.h"
#include "wf_launch.hpp"

namespace wf {

static __device__ __align__(256) char scratch[WF_DENSE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per device with that
// device current.  The array's name in host code is only a stand-in for the symbol.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_dense_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                                int N, int D, float scale, hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_dense(q, k, v, o, lse, BH, N, D, scale, WF_SOFTMAX_GUARDED, ws, s);
}

}  // namespace wf
