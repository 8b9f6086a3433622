// tsp_attn_forward_noalloc: the attention half of the layer (tsp_attn_forward)
// with its scratch memory in a fixed device array of the library instead of a
// caller workspace, for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that must not call hipMalloc, harnesses
// that forbid it).  The kernels are tsp_attn_forward's; only where their
// scratch lives differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

// The scratch array: Q, the attention output as a bf16 (hi, lo) pair, and the
// split partials of short sequences (tsp_workspace_size(.., TSP_WS_ATTN)
// bytes), at most TSP_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` is only
// a stand-in for the symbol: kernels receive the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[TSP_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];  // device address of `scratch` per device, resolved once

// The current device's address of `scratch` (resolved on the first call on
// that device, with that device current), or null on a HIP error.
void* scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= MAX_DEVICES) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" tsp_status tsp_attn_forward_noalloc(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                                               const uint16_t* const* wqkv, const uint16_t* const* wo,
                                               uint16_t* k_full, uint16_t* v_full, const uint16_t* residual,
                                               uint16_t* out, hipStream_t stream) {
  if (!plan || !dims) return TSP_ERR_INVALID_ARG;
  const size_t need = tsp_workspace_size(plan->n_local, dims, plan->D, TSP_WS_ATTN);
  // invalid dims or plan (no size): tsp_attn_forward's own checks return the
  // status, before anything is enqueued and before any HIP call
  if (need == 0) return tsp_attn_forward(plan, dims, x_local, wqkv, wo, k_full, v_full, residual, out, nullptr, 0, stream);
  if (need > (size_t)TSP_NOALLOC_SCRATCH_BYTES) return TSP_ERR_SCRATCH;
  hipError_t err;
  void* ws = scratch_ptr(&err);
  if (!ws) return TSP_ERR_HIP;
  return tsp_attn_forward(plan, dims, x_local, wqkv, wo, k_full, v_full, residual, out, ws,
                          (size_t)TSP_NOALLOC_SCRATCH_BYTES, stream);
}
