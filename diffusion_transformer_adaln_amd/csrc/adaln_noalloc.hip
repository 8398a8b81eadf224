// adaln_bwd_noalloc: the dense backward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  It is adaln_bwd with the workspace (the per-tile
// column partials) taken from a static device array of this library instead
// of a caller buffer: the same validation, kernels and results.
//
// The array `scratch` below is a device symbol; in host code its name is a
// host-side stand-in, not a device address, so host code never passes it to
// a kernel.  Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, on the entry point's first
// call there, and kept per device: each device holds its own copy at its own
// address until the process ends.  No hipMalloc, hipFree or allocating
// library call is made.  Nothing in the array has to start at zero (the
// backward writes every partial it later reads), and every call on one
// device shares that device's array, so calls that overlap in time on one
// device (different streams, or threads) race on it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/adaln.h"
#include "adaln_internal.hpp"

#define ADALN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) unsigned char scratch[ADALN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's address of `scratch` (looked up on first use).
adaln_status_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ADALN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ADALN_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ADALN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ADALN_OK;
}

}  // namespace

ADALN_EXPORT adaln_status_t adaln_bwd_noalloc(const void* dy, const void* x, const void* scale,
                                              const float* mean, const float* rstd, int64_t B,
                                              int64_t N, int64_t D, adaln_dtype_t dtype,
                                              hipStream_t stream, void* dx, void* dscale,
                                              void* dshift) {
  if (N < 0 || B < 1) return ADALN_ERR_INVALID_ARG;
  int64_t R = 0;
  if (N != 0 && B > INT64_MAX / N) return ADALN_ERR_UNSUPPORTED_SHAPE;
  R = B * N;
  // The workspace the problem needs (0 for sizes the backward rejects anyway,
  // which then fail its own validation below with their own code).
  const size_t need = adaln_bwd_workspace_size(B, R, D, dtype);
  if (need > ADALN_NOALLOC_SCRATCH_BYTES) return ADALN_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const adaln_status_t st = scratch_for_current_device(&ws);
  if (st != ADALN_OK) return st;
  return adaln::bwd_dense_with_workspace(dy, x, scale, mean, rstd, B, N, D, dtype, ws,
                                         ADALN_NOALLOC_SCRATCH_BYTES, stream, dx, dscale, dshift);
}
