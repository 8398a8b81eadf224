// C ABI of the fused AdaLN library: argument validation, path selection and
// launch.  Every check runs before anything is enqueued, so a validation
// error leaves all outputs untouched.  See include/adaln.h for the contract.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/adaln.h"
#include "adaln_internal.hpp"

#define ADALN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using adaln::BF16;
using adaln::F32;

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_cus[kMaxDevices] = {0};

// Compute units of the current device, cached per device.
hipError_t current_device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_cus[dev] > 0) { *cus = g_dev_cus[dev]; return hipSuccess; }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  g_dev_cus[dev] = n;
  *cus = n;
  return hipSuccess;
}

int64_t esize(adaln_dtype_t dt) { return dt == ADALN_BF16 ? 2 : 4; }

bool dtype_ok(adaln_dtype_t dt) { return dt == ADALN_F32 || dt == ADALN_BF16; }

// a*b (both >= 0) without int64 overflow
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Span {
  const void* p;
  int64_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  const uintptr_t a1 = a0 + static_cast<uintptr_t>(a.bytes), b1 = b0 + static_cast<uintptr_t>(b.bytes);
  return a0 < b1 && b0 < a1;
}

// any output overlapping any input, or two outputs overlapping
bool any_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Sizes {
  int64_t R, row_bytes_total, mod_bytes, stat_bytes;
  int64_t sum_bytes_f32;   // a [B, D] fp32 column-sum output
};

// Shared shape checks.  R = total rows.
adaln_status_t check_shape(int64_t B, int64_t R, int64_t D, adaln_dtype_t dt, Sizes* s) {
  if (!dtype_ok(dt)) return ADALN_ERR_UNSUPPORTED_DTYPE;
  if (B < 1 || R < 0 || D < 1) return ADALN_ERR_INVALID_ARG;
  if (D > ADALN_MAX_D) return ADALN_ERR_UNSUPPORTED_SHAPE;
  int64_t rd, rdb, bd, bdb, bd4, rs;
  if (!mul_ok(R, D, &rd) || !mul_ok(rd, esize(dt), &rdb) || !mul_ok(B, D, &bd) ||
      !mul_ok(bd, esize(dt), &bdb) || !mul_ok(bd, 4, &bd4) || !mul_ok(R, 4, &rs) ||
      rd > (INT64_MAX >> 8))
    return ADALN_ERR_UNSUPPORTED_SHAPE;
  s->R = R;
  s->row_bytes_total = rdb;
  s->mod_bytes = bdb;
  s->stat_bytes = rs;
  s->sum_bytes_f32 = bd4;
  return ADALN_OK;
}

adaln_status_t fwd_common(const void* x, const void* shift, const void* scale, float eps,
                          const int64_t* offsets, int64_t B, int64_t N, int64_t R, int64_t D,
                          adaln_dtype_t dtype, hipStream_t stream, void* y, float* mean,
                          float* rstd) {
  Sizes s;
  adaln_status_t st = check_shape(B, R, D, dtype, &s);
  if (st != ADALN_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f) return ADALN_ERR_INVALID_ARG;
  if (!shift || !scale) return ADALN_ERR_INVALID_ARG;
  if (R > 0 && (!x || !y || !mean || !rstd)) return ADALN_ERR_INVALID_ARG;
  const Span outs[] = {{y, s.row_bytes_total}, {mean, s.stat_bytes}, {rstd, s.stat_bytes}};
  const Span ins[] = {{x, s.row_bytes_total}, {shift, s.mod_bytes}, {scale, s.mod_bytes},
                      {offsets, offsets ? (B + 1) * 8 : 0}};
  if (any_alias(outs, 3, ins, 4)) return ADALN_ERR_ALIASING;
  if (R == 0) return ADALN_OK;

  int cus = 0;
  if (current_device_cus(&cus) != hipSuccess) return ADALN_ERR_HIP;
  const adaln::VecPlan vp = adaln::plan_vec(dtype, D, false);
  const bool vec = vp.ok && aligned16(x) && aligned16(y) && aligned16(shift) && aligned16(scale);
  const adaln::RowMap rm{B, R, N, offsets};
  const hipError_t e = adaln::launch_fwd(dtype, x, shift, scale, eps, rm, D, vec, vp, cus, stream,
                                         y, mean, rstd);
  return e == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// The backward entry points: the fused backward with column sums in the I/O
// type or in fp32, and the unfused two-pass ablation.
enum class BwdMode { kFused, kFusedF32Sums, kTwoPass };

adaln_status_t bwd_common(const void* dy, const void* x, const void* scale, const float* mean,
                          const float* rstd, const int64_t* offsets, int64_t B, int64_t N,
                          int64_t R, int64_t D, adaln_dtype_t dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, void* dx, void* dscale,
                          void* dshift, BwdMode mode) {
  Sizes s;
  adaln_status_t st = check_shape(B, R, D, dtype, &s);
  if (st != ADALN_OK) return st;
  if (!scale || !dscale || !dshift) return ADALN_ERR_INVALID_ARG;
  if (R > 0 && (!dy || !x || !mean || !rstd || !dx)) return ADALN_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return ADALN_ERR_INVALID_ARG;

  int cus = 0;
  if (current_device_cus(&cus) != hipSuccess) return ADALN_ERR_HIP;
  const adaln::WorkspaceLayout wl =
      adaln::bwd_workspace_layout(B, R, D, cus, offsets != nullptr, N);
  if (workspace_bytes < wl.total) return ADALN_ERR_WORKSPACE_TOO_SMALL;
  // one workgroup per tile; up to B * ceil(D/16) finish workgroups
  const int64_t col_blocks = (D + 15) / 16;
  if (wl.tiles_max > INT32_MAX || B > INT32_MAX / col_blocks) return ADALN_ERR_UNSUPPORTED_SHAPE;

  const bool sums_f32 = mode == BwdMode::kFusedF32Sums;
  const int64_t sum_bytes = sums_f32 ? s.sum_bytes_f32 : s.mod_bytes;
  const Span outs[] = {{dx, s.row_bytes_total},
                       {dscale, sum_bytes},
                       {dshift, sum_bytes},
                       {workspace, static_cast<int64_t>(wl.total)}};
  const Span ins[] = {{dy, s.row_bytes_total}, {x, s.row_bytes_total}, {scale, s.mod_bytes},
                      {mean, s.stat_bytes},    {rstd, s.stat_bytes},
                      {offsets, offsets ? (B + 1) * 8 : 0}};
  if (any_alias(outs, 4, ins, 6)) return ADALN_ERR_ALIASING;

  const adaln::VecPlan vp = adaln::plan_vec(dtype, D, true, offsets != nullptr, B);
  const bool vec = vp.ok && aligned16(dy) && aligned16(x) && aligned16(dx) && aligned16(scale);
  const bool twopass = mode == BwdMode::kTwoPass;
  if (twopass && !vec) return ADALN_ERR_UNSUPPORTED_SHAPE;
  char* ws = static_cast<char*>(workspace);
  adaln::Tiling tl{wl.tile_rows, wl.tiles_max, wl.tiles_alloc,
                   offsets ? reinterpret_cast<int64_t*>(ws + wl.tile_start_off) : nullptr, 1};
  float* partial = reinterpret_cast<float*>(ws + wl.partial_off);
  const adaln::RowMap rm{B, R, N, offsets};
  const hipError_t e =
      twopass ? adaln::launch_bwd_twopass(dtype, dy, x, scale, mean, rstd, rm, D, vp, tl, partial,
                                          stream, dx, dscale, dshift)
              : adaln::launch_bwd(dtype, dy, x, scale, mean, rstd, rm, D, vec, vp, tl, partial,
                                  stream, dx, dscale, dshift, sums_f32);
  return e == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

}  // namespace

namespace adaln {
// The dense backward with a workspace the caller (or the no-allocation entry
// point's static scratch) provides; adaln_bwd's body.
adaln_status_t bwd_dense_with_workspace(const void* dy, const void* x, const void* scale,
                                        const float* mean, const float* rstd, int64_t B, int64_t N,
                                        int64_t D, adaln_dtype_t dtype, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream, void* dx,
                                        void* dscale, void* dshift) {
  if (N < 0 || B < 1) return ADALN_ERR_INVALID_ARG;
  int64_t R;
  if (!mul_ok(B, N, &R)) return ADALN_ERR_UNSUPPORTED_SHAPE;
  return bwd_common(dy, x, scale, mean, rstd, nullptr, B, N, R, D, dtype, workspace,
                    workspace_bytes, stream, dx, dscale, dshift, BwdMode::kFused);
}
}  // namespace adaln

ADALN_EXPORT adaln_status_t adaln_fwd(const void* x, const void* shift, const void* scale,
                                      float eps, int64_t B, int64_t N, int64_t D,
                                      adaln_dtype_t dtype, hipStream_t stream, void* y,
                                      float* mean, float* rstd) {
  if (N < 0 || B < 1) return ADALN_ERR_INVALID_ARG;
  int64_t R;
  if (!mul_ok(B, N, &R)) return ADALN_ERR_UNSUPPORTED_SHAPE;
  return fwd_common(x, shift, scale, eps, nullptr, B, N, R, D, dtype, stream, y, mean, rstd);
}

ADALN_EXPORT adaln_status_t adaln_fwd_varlen(const void* x, const void* shift, const void* scale,
                                             float eps, const int64_t* offsets_dev, int64_t B,
                                             int64_t total_rows, int64_t D, adaln_dtype_t dtype,
                                             hipStream_t stream, void* y, float* mean,
                                             float* rstd) {
  if (!offsets_dev) return ADALN_ERR_INVALID_ARG;
  return fwd_common(x, shift, scale, eps, offsets_dev, B, 0, total_rows, D, dtype, stream, y,
                    mean, rstd);
}

ADALN_EXPORT size_t adaln_bwd_workspace_size(int64_t B, int64_t total_rows, int64_t D,
                                             adaln_dtype_t dtype) {
  Sizes s;
  if (check_shape(B, total_rows, D, dtype, &s) != ADALN_OK) return 0;
  int cus = 0;
  if (current_device_cus(&cus) != hipSuccess) return 0;
  return adaln::bwd_workspace_bytes(B, total_rows, D, cus);
}

ADALN_EXPORT adaln_status_t adaln_bwd(const void* dy, const void* x, const void* scale,
                                      const float* mean, const float* rstd, int64_t B, int64_t N,
                                      int64_t D, adaln_dtype_t dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, void* dx,
                                      void* dscale, void* dshift) {
  return adaln::bwd_dense_with_workspace(dy, x, scale, mean, rstd, B, N, D, dtype, workspace,
                                         workspace_bytes, stream, dx, dscale, dshift);
}

ADALN_EXPORT adaln_status_t adaln_bwd_varlen(const void* dy, const void* x, const void* scale,
                                             const float* mean, const float* rstd,
                                             const int64_t* offsets_dev, int64_t B,
                                             int64_t total_rows, int64_t D, adaln_dtype_t dtype,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream, void* dx, void* dscale,
                                             void* dshift) {
  if (!offsets_dev) return ADALN_ERR_INVALID_ARG;
  return bwd_common(dy, x, scale, mean, rstd, offsets_dev, B, 0, total_rows, D, dtype, workspace,
                    workspace_bytes, stream, dx, dscale, dshift, BwdMode::kFused);
}

ADALN_EXPORT adaln_status_t adaln_bwd_f32sums(const void* dy, const void* x, const void* scale,
                                              const float* mean, const float* rstd, int64_t B,
                                              int64_t N, int64_t D, adaln_dtype_t dtype,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, void* dx, float* dscale,
                                              float* dshift) {
  if (N < 0 || B < 1) return ADALN_ERR_INVALID_ARG;
  int64_t R;
  if (!mul_ok(B, N, &R)) return ADALN_ERR_UNSUPPORTED_SHAPE;
  return bwd_common(dy, x, scale, mean, rstd, nullptr, B, N, R, D, dtype, workspace,
                    workspace_bytes, stream, dx, dscale, dshift, BwdMode::kFusedF32Sums);
}

ADALN_EXPORT adaln_status_t adaln_bwd_varlen_f32sums(const void* dy, const void* x,
                                                     const void* scale, const float* mean,
                                                     const float* rstd,
                                                     const int64_t* offsets_dev, int64_t B,
                                                     int64_t total_rows, int64_t D,
                                                     adaln_dtype_t dtype, void* workspace,
                                                     size_t workspace_bytes, hipStream_t stream,
                                                     void* dx, float* dscale, float* dshift) {
  if (!offsets_dev) return ADALN_ERR_INVALID_ARG;
  return bwd_common(dy, x, scale, mean, rstd, offsets_dev, B, 0, total_rows, D, dtype, workspace,
                    workspace_bytes, stream, dx, dscale, dshift, BwdMode::kFusedF32Sums);
}

ADALN_EXPORT adaln_status_t adaln_bwd_twopass(const void* dy, const void* x, const void* scale,
                                              const float* mean, const float* rstd, int64_t B,
                                              int64_t N, int64_t D, adaln_dtype_t dtype,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, void* dx, void* dscale,
                                              void* dshift) {
  if (N < 0 || B < 1) return ADALN_ERR_INVALID_ARG;
  int64_t R;
  if (!mul_ok(B, N, &R)) return ADALN_ERR_UNSUPPORTED_SHAPE;
  return bwd_common(dy, x, scale, mean, rstd, nullptr, B, N, R, D, dtype, workspace,
                    workspace_bytes, stream, dx, dscale, dshift, BwdMode::kTwoPass);
}

ADALN_EXPORT const char* adaln_status_str(adaln_status_t status) {
  switch (status) {
    case ADALN_OK: return "ADALN_OK";
    case ADALN_ERR_INVALID_ARG: return "ADALN_ERR_INVALID_ARG";
    case ADALN_ERR_UNSUPPORTED_DTYPE: return "ADALN_ERR_UNSUPPORTED_DTYPE";
    case ADALN_ERR_UNSUPPORTED_SHAPE: return "ADALN_ERR_UNSUPPORTED_SHAPE";
    case ADALN_ERR_WORKSPACE_TOO_SMALL: return "ADALN_ERR_WORKSPACE_TOO_SMALL";
    case ADALN_ERR_ALIASING: return "ADALN_ERR_ALIASING";
    case ADALN_ERR_HIP: return "ADALN_ERR_HIP";
  }
  return "ADALN_ERR_UNKNOWN";
}

ADALN_EXPORT int adaln_abi_version(void) { return ADALN_ABI_VERSION; }
