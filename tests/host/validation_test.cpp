// Host-only test of the C ABI's argument validation (include/adaln.h, "Errors"):
// the real dispatcher (csrc/adaln_api.cpp) and planning code (csrc/adaln_plan.cpp)
// linked against stub launchers that count launches and a stub device query
// that reports one 256-CU device.  Built with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_validation.py.
//
// Checks, for every entry point: each documented error code is returned for
// its cause, a failing call launches nothing, a valid call launches exactly
// once with the shape (and, for the backward, the column-sum type) it was
// given, fp32 column sums are sized as such for the aliasing check, adaln_bwd_workspace_size() is enough for
// both backward entry points, and each of them accepts exactly its own
// workspace layout and rejects one byte less.  Also the host planner's
// invariants that the kernels rely on (row layouts for every D, tilings).

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <algorithm>
#include <vector>

#include "adaln.h"
#include "../../diffusion_transformer_adaln_amd/csrc/adaln_internal.hpp"

// ---------------------------------------------------------------------------
// stubs: one device with 256 compute units; launchers record their calls
// ---------------------------------------------------------------------------
static int g_launches = 0;
static adaln::RowMap g_rm{};
static int64_t g_D = 0;
static adaln::Tiling g_tl{};
static bool g_sums_f32 = false;

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *v = 256;
  return hipSuccess;
}

namespace adaln {
hipError_t launch_fwd(int, const void*, const void*, const void*, float, const RowMap& rm, int64_t D,
                      bool, const VecPlan&, int, hipStream_t, void*, float*, float*) {
  ++g_launches; g_rm = rm; g_D = D;
  return hipSuccess;
}
hipError_t launch_bwd(int, const void*, const void*, const void*, const float*, const float*,
                      const RowMap& rm, int64_t D, bool, const VecPlan&, const Tiling& tl, float*,
                      hipStream_t, void*, void*, void*, bool sums_f32) {
  ++g_launches; g_rm = rm; g_D = D; g_tl = tl; g_sums_f32 = sums_f32;
  return hipSuccess;
}
hipError_t launch_bwd_twopass(int, const void*, const void*, const void*, const float*,
                              const float*, const RowMap& rm, int64_t D, const VecPlan&,
                              const Tiling& tl, float*, hipStream_t, void*, void*, void*) {
  ++g_launches; g_rm = rm; g_D = D; g_tl = tl;
  return hipSuccess;
}
}  // namespace adaln

// ---------------------------------------------------------------------------
// checks
// ---------------------------------------------------------------------------
static int g_failures = 0, g_checks = 0;

#define EXPECT(cond, ...)                                          \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(cond)) {                                                 \
      ++g_failures;                                                \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__);             \
      std::printf(__VA_ARGS__);                                    \
      std::printf("\n");                                           \
    }                                                              \
  } while (0)

// A call that must fail with `want` and launch nothing.
#define REJECT(want, call)                                                                  \
  do {                                                                                      \
    const int before_ = g_launches;                                                         \
    const adaln_status_t got_ = (call);                                                     \
    EXPECT(got_ == (want), "%s: got %s, want %s", #call, adaln_status_str(got_),           \
           adaln_status_str(want));                                                         \
    EXPECT(g_launches == before_, "%s: launched on error", #call);                          \
  } while (0)

// A call that must succeed with exactly `n` launches.
#define ACCEPT(n, call)                                                                     \
  do {                                                                                      \
    const int before_ = g_launches;                                                         \
    const adaln_status_t got_ = (call);                                                     \
    EXPECT(got_ == ADALN_OK, "%s: got %s", #call, adaln_status_str(got_));                 \
    EXPECT(g_launches == before_ + (n), "%s: %d launches, want %d", #call,                  \
           g_launches - before_, (n));                                                      \
  } while (0)

// Fake device addresses: validation never dereferences them.  Each buffer
// gets its own 64 GiB region so nothing overlaps unless a test says so.
static void* at(int region) { return reinterpret_cast<void*>(static_cast<uintptr_t>(region) << 36); }
static float* fat(int region) { return static_cast<float*>(at(region)); }

static void test_forward() {
  const int64_t B = 2, N = 100, D = 1152;
  void *x = at(1), *sh = at(2), *sc = at(3), *y = at(4);
  float *m = fat(5), *r = fat(6);
  const adaln_dtype_t bf = ADALN_BF16;

  ACCEPT(1, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, y, m, r));
  EXPECT(g_rm.B == B && g_rm.R == B * N && g_rm.N == N && g_rm.offsets == nullptr && g_D == D,
         "forward launched with the wrong shape");
  ACCEPT(0, adaln_fwd(x, sh, sc, 1e-6f, B, 0, D, bf, nullptr, y, m, r));   // empty batch
  ACCEPT(0, adaln_fwd(nullptr, sh, sc, 1e-6f, B, 0, D, bf, nullptr, nullptr, nullptr, nullptr));
  ACCEPT(1, adaln_fwd(x, sh, sc, 0.0f, B, N, D, ADALN_F32, nullptr, y, m, r));

  REJECT(ADALN_ERR_UNSUPPORTED_DTYPE, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, (adaln_dtype_t)7, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, 0, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, B, -1, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, B, N, 0, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_UNSUPPORTED_SHAPE, adaln_fwd(x, sh, sc, 1e-6f, B, N, ADALN_MAX_D + 1, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_UNSUPPORTED_SHAPE, adaln_fwd(x, sh, sc, 1e-6f, INT64_MAX / 4, 8, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_UNSUPPORTED_SHAPE, adaln_fwd(x, sh, sc, 1e-6f, 1, INT64_MAX / 1024, 4096, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, -1e-6f, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, NAN, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, INFINITY, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(nullptr, sh, sc, 1e-6f, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, nullptr, sc, 1e-6f, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, nullptr, 1e-6f, B, N, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, nullptr, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, y, nullptr, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, y, m, nullptr));
  // aliasing: y over x (in place), y over shift, mean over rstd, y ending one byte into x
  REJECT(ADALN_ERR_ALIASING, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, x, m, r));
  REJECT(ADALN_ERR_ALIASING, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, sh, m, r));
  REJECT(ADALN_ERR_ALIASING, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, y, m, m + 1));
  char* xb = static_cast<char*>(x);
  const int64_t bytes = B * N * D * 2;
  REJECT(ADALN_ERR_ALIASING, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, xb - bytes + 1, m, r));
  ACCEPT(1, adaln_fwd(x, sh, sc, 1e-6f, B, N, D, bf, nullptr, xb - bytes, m, r));   // adjacent is fine
}

static void test_forward_varlen() {
  const int64_t B = 3, R = 77, D = 3072;
  void *x = at(1), *sh = at(2), *sc = at(3), *y = at(4);
  float *m = fat(5), *r = fat(6);
  const int64_t* off = static_cast<const int64_t*>(at(7));
  const adaln_dtype_t bf = ADALN_BF16;
  ACCEPT(1, adaln_fwd_varlen(x, sh, sc, 1e-6f, off, B, R, D, bf, nullptr, y, m, r));
  EXPECT(g_rm.B == B && g_rm.R == R && g_rm.offsets == off && g_D == D, "varlen forward launched with the wrong shape");
  ACCEPT(0, adaln_fwd_varlen(x, sh, sc, 1e-6f, off, B, 0, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd_varlen(x, sh, sc, 1e-6f, nullptr, B, R, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd_varlen(x, sh, sc, 1e-6f, off, 0, R, D, bf, nullptr, y, m, r));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_fwd_varlen(x, sh, sc, 1e-6f, off, B, -5, D, bf, nullptr, y, m, r));
  // the offsets are an input: an output over them is aliasing
  REJECT(ADALN_ERR_ALIASING, adaln_fwd_varlen(x, sh, sc, 1e-6f, off, B, R, D, bf, nullptr, y,
                                              reinterpret_cast<float*>(const_cast<int64_t*>(off)), r));
}

static void test_backward() {
  const int64_t B = 2, N = 4096, D = 3072;
  void *dy = at(1), *x = at(2), *sc = at(3), *dx = at(4), *dsc = at(5), *dsh = at(6), *ws = at(9);
  const float *m = fat(7), *r = fat(8);
  const adaln_dtype_t bf = ADALN_BF16;
  const size_t need = adaln_bwd_workspace_size(B, B * N, D, bf);
  EXPECT(need > 0, "workspace size query returned 0 for a valid shape");

  for (int pass = 0; pass < 2; ++pass) {
    auto call = [&](void* dy_, void* x_, void* sc_, const float* m_, const float* r_, int64_t B_, int64_t N_,
                    int64_t D_, adaln_dtype_t dt, void* ws_, size_t wsb, void* dx_, void* dsc_, void* dsh_) {
      return pass == 0 ? adaln_bwd(dy_, x_, sc_, m_, r_, B_, N_, D_, dt, ws_, wsb, nullptr, dx_, dsc_, dsh_)
                       : adaln_bwd_twopass(dy_, x_, sc_, m_, r_, B_, N_, D_, dt, ws_, wsb, nullptr, dx_, dsc_, dsh_);
    };
    ACCEPT(1, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dx, dsc, dsh));
    EXPECT(g_rm.B == B && g_rm.R == B * N && g_rm.N == N && g_D == D && g_tl.tiles_max > 0 &&
               g_tl.tiles_max <= g_tl.tiles_alloc && g_tl.tile_start == nullptr,
           "backward launched with the wrong shape or tiling");
    const size_t own = adaln::bwd_workspace_layout(B, B * N, D, 256, false, N).total;
    EXPECT(own <= need, "dense layout larger than the size query");
    ACCEPT(1, call(dy, x, sc, m, r, B, N, D, bf, ws, own, dx, dsc, dsh));
    REJECT(ADALN_ERR_WORKSPACE_TOO_SMALL, call(dy, x, sc, m, r, B, N, D, bf, ws, own - 1, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, N, D, bf, nullptr, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, N, D, bf, static_cast<char*>(ws) + 8, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_UNSUPPORTED_DTYPE, call(dy, x, sc, m, r, B, N, D, (adaln_dtype_t)-1, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, 0, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, -1, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_UNSUPPORTED_SHAPE, call(dy, x, sc, m, r, B, N, ADALN_MAX_D * 2, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(nullptr, x, sc, m, r, B, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, nullptr, sc, m, r, B, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, nullptr, m, r, B, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, nullptr, r, B, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, nullptr, B, N, D, bf, ws, need, dx, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dsc, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dx, nullptr, dsh));
    REJECT(ADALN_ERR_INVALID_ARG, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dx, dsc, nullptr));
    // aliasing: dx over dy, dscale over dshift, dshift inside the workspace, workspace over x
    REJECT(ADALN_ERR_ALIASING, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dy, dsc, dsh));
    REJECT(ADALN_ERR_ALIASING, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dx, dsc, static_cast<char*>(dsc) + 2));
    REJECT(ADALN_ERR_ALIASING, call(dy, x, sc, m, r, B, N, D, bf, ws, need, dx, dsc, static_cast<char*>(ws) + 2));
    REJECT(ADALN_ERR_ALIASING, call(dy, x, sc, m, r, B, N, D, bf, x, need, dx, dsc, dsh));
  }
  // N == 0: the backward still runs (its finish writes zero dscale/dshift)
  ACCEPT(1, adaln_bwd(nullptr, nullptr, sc, nullptr, nullptr, B, 0, D, bf, ws, adaln_bwd_workspace_size(B, 0, D, bf),
                      nullptr, nullptr, dsc, dsh));

  // fp32 column sums: the same checks, the flag reaches the launcher, and the
  // sums are 4*B*D-byte buffers for the aliasing check whatever dtype is
  float *fsc = fat(5), *fsh = fat(6);
  ACCEPT(1, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, fsc, fsh));
  EXPECT(g_sums_f32 && g_rm.R == B * N && g_rm.offsets == nullptr && g_D == D,
         "f32-sums backward launched with the wrong shape or flag");
  ACCEPT(1, adaln_bwd(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, dsc, dsh));
  EXPECT(!g_sums_f32, "adaln_bwd launched with fp32 sums");
  float* after_bf16 = reinterpret_cast<float*>(static_cast<char*>(dsc) + B * D * 2);   // inside fp32 dscale
  ACCEPT(1, adaln_bwd(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, dsc, after_bf16));
  REJECT(ADALN_ERR_ALIASING, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, fsc, after_bf16));
  ACCEPT(1, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, fsc, fsc + B * D));
  REJECT(ADALN_ERR_ALIASING, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, fsc,
                                               fsc + B * D - 1));
  REJECT(ADALN_ERR_ALIASING, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx,
                                               static_cast<float*>(sc), fsh));
  REJECT(ADALN_ERR_WORKSPACE_TOO_SMALL, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws,
                                                          adaln::bwd_workspace_layout(B, B * N, D, 256, false, N).total - 1,
                                                          nullptr, dx, fsc, fsh));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, bf, ws, need, nullptr, dx, nullptr, fsh));
  REJECT(ADALN_ERR_INVALID_ARG, adaln_bwd_f32sums(dy, x, sc, m, r, B, -1, D, bf, ws, need, nullptr, dx, fsc, fsh));
  REJECT(ADALN_ERR_UNSUPPORTED_DTYPE, adaln_bwd_f32sums(dy, x, sc, m, r, B, N, D, (adaln_dtype_t)3, ws, need,
                                                        nullptr, dx, fsc, fsh));
  REJECT(ADALN_ERR_UNSUPPORTED_SHAPE, adaln_bwd_f32sums(dy, x, sc, m, r, INT64_MAX / 8, 1, 4096, bf, ws, need,
                                                        nullptr, dx, fsc, fsh));
  ACCEPT(1, adaln_bwd_f32sums(nullptr, nullptr, sc, nullptr, nullptr, B, 0, D, ADALN_F32, ws,
                              adaln_bwd_workspace_size(B, 0, D, ADALN_F32), nullptr, nullptr, fsc, fsh));
  // workspace query: invalid sizes give 0
  EXPECT(adaln_bwd_workspace_size(0, 10, D, bf) == 0, "B = 0 accepted by the size query");
  EXPECT(adaln_bwd_workspace_size(B, -1, D, bf) == 0, "negative rows accepted by the size query");
  EXPECT(adaln_bwd_workspace_size(B, 10, 0, bf) == 0, "D = 0 accepted by the size query");
  EXPECT(adaln_bwd_workspace_size(B, 10, D, (adaln_dtype_t)9) == 0, "bad dtype accepted by the size query");
}

static void test_backward_varlen() {
  // the size query covers the packed layout as well as the dense one
  const adaln_dtype_t bf = ADALN_BF16;
  void *dy = at(1), *x = at(2), *sc = at(3), *dx = at(4), *dsc = at(5), *dsh = at(6), *ws = at(9);
  const float *m = fat(7), *r = fat(8);
  const int64_t* off = static_cast<const int64_t*>(at(10));
  const int64_t shapes[][3] = {{277, 229368, 3072}, {1, 18900, 5120}, {5, 3, 128}, {300, 300, 1152}, {2, 1, 8}};
  for (const auto& s : shapes) {
    const int64_t B = s[0], R = s[1], D = s[2];
    const size_t need = adaln_bwd_workspace_size(B, R, D, bf);
    ACCEPT(1, adaln_bwd_varlen(dy, x, sc, m, r, off, B, R, D, bf, ws, need, nullptr, dx, dsc, dsh));
    EXPECT(g_rm.offsets == off && g_tl.tile_start != nullptr && g_tl.tiles_max <= g_tl.tiles_alloc,
           "packed backward tiling inconsistent for B=%lld R=%lld", (long long)B, (long long)R);
    const size_t own = adaln::bwd_workspace_layout(B, R, D, 256, true, 0).total;
    EXPECT(own <= need, "packed layout larger than the size query");
    REJECT(ADALN_ERR_WORKSPACE_TOO_SMALL,
           adaln_bwd_varlen(dy, x, sc, m, r, off, B, R, D, bf, ws, own - 1, nullptr, dx, dsc, dsh));
    if (R % B == 0) {
      ACCEPT(1, adaln_bwd(dy, x, sc, m, r, B, R / B, D, bf, ws, need, nullptr, dx, dsc, dsh));
    }
  }
  REJECT(ADALN_ERR_INVALID_ARG, adaln_bwd_varlen(dy, x, sc, m, r, nullptr, 2, 10, 64, bf, ws, 1 << 20, nullptr, dx, dsc, dsh));

  // fp32 column sums of packed samples
  float *fsc = fat(5), *fsh = fat(6);
  const int64_t B = 277, R = 229368, D = 3072;
  const size_t need = adaln_bwd_workspace_size(B, R, D, bf);
  ACCEPT(1, adaln_bwd_varlen_f32sums(dy, x, sc, m, r, off, B, R, D, bf, ws, need, nullptr, dx, fsc, fsh));
  EXPECT(g_sums_f32 && g_rm.offsets == off && g_tl.tile_start != nullptr && g_rm.R == R,
         "packed f32-sums backward launched with the wrong shape or flag");
  REJECT(ADALN_ERR_INVALID_ARG, adaln_bwd_varlen_f32sums(dy, x, sc, m, r, nullptr, B, R, D, bf, ws, need, nullptr,
                                                         dx, fsc, fsh));
  REJECT(ADALN_ERR_ALIASING, adaln_bwd_varlen_f32sums(dy, x, sc, m, r, off, B, R, D, bf, ws, need, nullptr, dx, fsc,
                                                      fsc + B * D - 4));
  REJECT(ADALN_ERR_ALIASING, adaln_bwd_varlen_f32sums(dy, x, sc, m, r, off, B, R, D, bf, ws, need, nullptr, dx, fsc,
                                                      reinterpret_cast<float*>(const_cast<int64_t*>(off))));
  REJECT(ADALN_ERR_WORKSPACE_TOO_SMALL,
         adaln_bwd_varlen_f32sums(dy, x, sc, m, r, off, B, R, D, bf, ws,
                                  adaln::bwd_workspace_layout(B, R, D, 256, true, 0).total - 1, nullptr, dx, fsc, fsh));
}

static void test_status_strings() {
  for (int s = 0; s <= 6; ++s) EXPECT(adaln_status_str((adaln_status_t)s) != nullptr, "null status string");
  EXPECT(adaln_status_str((adaln_status_t)42) != nullptr, "null string for an unknown code");
  EXPECT(adaln_abi_version() == ADALN_ABI_VERSION, "ABI version mismatch");
}

// The planner's invariants that the kernels rely on, for every row width up
// to the largest supported D: a vector plan covers the row exactly with lane
// groups the reductions handle, fits one workgroup and its LDS, and carries
// two rows per slot only where the forward instantiates that; the backward's
// tiling puts every tile inside the partial-sum buffer it sizes.
static void test_plans() {
  for (int dt : {adaln::F32, adaln::BF16}) {
    const int64_t epv = dt == adaln::BF16 ? 8 : 4;
    for (int64_t D = 1; D <= ADALN_MAX_D; ++D) {
      for (int dir = 0; dir < 4; ++dir) {   // forward, dense backward, packed backward (few, many samples)
        const bool bwd = dir > 0;
        const adaln::VecPlan p = adaln::plan_vec(dt, D, bwd, dir >= 2, dir == 3 ? 277 : 4);
        if (!p.ok) continue;   // the general kernels take these widths
        const int64_t V = D / epv;
        const bool shape_ok = p.vpt >= 1 && p.vpt <= (bwd ? adaln::BWD_MAX_VPT : adaln::FWD_MAX_VPT) &&
                              D % epv == 0 && static_cast<int64_t>(p.vpt) * p.lpr == V && p.lpr % 16 == 0;
        const bool wg_ok = p.nt >= p.lpr && p.nt % p.lpr == 0 && p.nt % 64 == 0 && p.nt <= adaln::VEC_MAX_NT;
        const bool rif_ok = bwd ? p.rif == adaln::BWD_RIF
                                : (p.rif == 1 || (p.rif == 2 && p.vpt <= adaln::FWD_RIF2_MAX_VPT));
        const bool lds_ok = adaln::vec_lds_bytes(p, D, bwd) <= 65536;
        EXPECT(shape_ok && wg_ok && rif_ok && lds_ok, "plan dtype %d D %lld dir %d: vpt %d lpr %d nt %d rif %d",
               dt, (long long)D, dir, p.vpt, p.lpr, p.nt, p.rif);
      }
    }
  }
  // the workloads' row widths, and the widest rows the GPU tests use, are vectorised
  const struct { int dt; int64_t D; } want[] = {{adaln::F32, 128}, {adaln::BF16, 1152}, {adaln::BF16, 3072},
                                               {adaln::BF16, 5120}, {adaln::BF16, 16384}, {adaln::F32, 4096}};
  for (const auto& w : want)
    for (int dir = 0; dir < 4; ++dir)
      EXPECT(adaln::plan_vec(w.dt, w.D, dir > 0, dir >= 2, dir == 3 ? 277 : 4).ok,
             "no vector plan for dtype %d D %lld dir %d", w.dt,
             (long long)w.D, dir);
  const int64_t Bs[] = {1, 2, 3, 8, 277};
  const int64_t Ns[] = {0, 1, 2, 3, 5, 64, 100, 512, 1023, 4096, 18900, 64000};
  const int cus_list[] = {1, 80, 256, 304};
  for (int cus : cus_list)
    for (int64_t B : Bs)
      for (int64_t N : Ns)
        for (int64_t D : {int64_t(8), int64_t(1152), int64_t(5120)}) {
          const int64_t R = B * N;
          for (int varlen = 0; varlen < 2; ++varlen) {
            const adaln::WorkspaceLayout w = adaln::bwd_workspace_layout(B, R, D, cus, varlen, N);
            const int64_t dense_tiles = B * ((N + w.tile_rows - 1) / w.tile_rows);
            const size_t chunks = static_cast<size_t>((D + adaln::PCOLS - 1) / adaln::PCOLS);
            const bool ok =
                w.tile_rows >= 1 && (R == 0 || w.tile_rows >= 4) &&
                w.tiles_alloc >= (R + w.tile_rows - 1) / w.tile_rows + B &&   // any split into B samples
                w.tiles_max <= w.tiles_alloc && (varlen || w.tiles_max == dense_tiles) &&
                w.partial_off % 256 == 0 && w.partial_off >= static_cast<size_t>(B + 1) * 8 &&
                w.total >= w.partial_off + chunks * static_cast<size_t>(w.tiles_alloc) * 2 * adaln::PCOLS * 4 &&
                adaln::bwd_workspace_bytes(B, R, D, cus) >= w.total;
            EXPECT(ok, "tiling B %lld N %lld D %lld cus %d varlen %d: tile_rows %lld tiles %lld/%lld", (long long)B,
                   (long long)N, (long long)D, cus, varlen, (long long)w.tile_rows, (long long)w.tiles_max,
                   (long long)w.tiles_alloc);
          }
        }
}

// Device offsets are trusted but clamped where the kernels read them: every
// sample's clamped span lies inside [0, R], and the packed backward's tile
// table (per-sample tile counts from the clamped spans, prefix sums capped at
// the partials' capacity, as the prologue computes it), mapped to rows the
// way the row pass maps them (tile k of a sample takes rows k, k + tiles, ...),
// never reaches a row outside [0, R) or a tile at or past tiles_alloc, for
// malformed tables too (negative, past R, decreasing, overlapping).
static void test_offset_clamp() {
  EXPECT(adaln::clamp_row(-5, 10) == 0 && adaln::clamp_row(11, 10) == 10 && adaln::clamp_row(7, 10) == 7,
         "clamp_row");
  const int64_t R = 1000, D = 64;
  const int cus = 256;
  const std::vector<std::vector<int64_t>> tables = {
      {0, 100, 1000},                      // well formed
      {-50, 400, 2000},                    // ends outside [0, R]
      {0, 900, 100, 1000},                 // decreasing
      {0, 1000, 0, 1000, 0, 1000},         // overlapping samples
      {5000, -7, 3000, 1000},              // nothing sensible
      {INT64_MIN, INT64_MAX},
  };
  for (const auto& o : tables) {
    const int64_t B = static_cast<int64_t>(o.size()) - 1;
    const adaln::WorkspaceLayout w = adaln::bwd_workspace_layout(B, R, D, cus, true, 0);
    int64_t start = 0;
    bool ok = true;
    for (int64_t b = 0; b < B; ++b) {
      const adaln::RowSpan sp = adaln::clamped_span(o[b], o[b + 1], R);
      ok = ok && sp.lo >= 0 && sp.n >= 0 && sp.lo + sp.n <= R;
      const int64_t cnt = sp.n > 0 ? (sp.n + w.tile_rows - 1) / w.tile_rows : 0;
      const int64_t t0 = start < w.tiles_alloc ? start : w.tiles_alloc;
      const int64_t t1 = start + cnt < w.tiles_alloc ? start + cnt : w.tiles_alloc;
      start += cnt;
      const int64_t tiles = t1 - t0;
      for (int64_t k = 0; k < tiles; ++k)
        for (int64_t r = sp.lo + k; r < sp.lo + sp.n; r += tiles) ok = ok && r >= 0 && r < R;
      ok = ok && t1 <= w.tiles_alloc && t0 <= t1;
    }
    EXPECT(ok, "offset table of %lld samples leaves [0, R) or the tile capacity", (long long)B);
  }
}

// Packed batches of at most 64 samples number their tiles without the
// prologue's table: a wave holds each sample's capped exclusive prefix
// (lane i: sample i) and a tile's sample is the highest lane whose prefix is
// <= t (a ballot), a tile at or past the capped total being spare.  That
// lookup must agree with the binary search over the prologue's table for
// every tile, empty and malformed samples included.
static void test_wave_tile_lookup() {
  const int64_t R = 5000, D = 256;
  const int cus = 256;
  std::vector<std::vector<int64_t>> tables = {
      {0, 5000}, {0, 0, 5000}, {0, 5000, 5000}, {0, 1, 2, 3, 4}, {0, 100, 100, 100, 4000, 5000},
      {-50, 400, 9000}, {0, 900, 100, 1000}, {0, 5000, 0, 5000, 0, 5000}, {INT64_MIN, INT64_MAX}};
  uint64_t seed = 12345;
  auto next = [&seed]() { seed = seed * 6364136223846793005ull + 1442695040888963407ull; return seed >> 33; };
  for (int B : {1, 2, 5, 17, 63, 64}) {
    std::vector<int64_t> o(B + 1, 0);
    for (int b = 1; b <= B; ++b) o[b] = o[b - 1] + static_cast<int64_t>(next() % 3 == 0 ? 0 : next() % 300);
    tables.push_back(o);
  }
  for (const auto& o : tables) {
    const int64_t B = static_cast<int64_t>(o.size()) - 1;
    const adaln::WorkspaceLayout w = adaln::bwd_workspace_layout(B, R, D, cus, true, 0);
    const int64_t TA = w.tiles_alloc;
    // the prologue's table
    std::vector<int64_t> start(B + 1);
    int64_t carry = 0;
    std::vector<int64_t> excl(B), incl(B);
    for (int64_t b = 0; b < B; ++b) {
      const int64_t n = adaln::clamped_span(o[b], o[b + 1], R).n;
      const int64_t cnt = n > 0 ? (n + w.tile_rows - 1) / w.tile_rows : 0;
      start[b] = carry < TA ? carry : TA;
      excl[b] = start[b];
      carry += cnt;
      incl[b] = carry < TA ? carry : TA;
    }
    start[B] = carry < TA ? carry : TA;
    bool ok = true;
    for (int64_t t = 0; t < TA + 3; ++t) {
      const bool spare_table = t >= start[B];
      const bool spare_wave = t >= incl[B - 1];
      ok = ok && spare_table == spare_wave;
      if (spare_table) continue;
      int64_t lo = 0, hi = B;
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (start[mid] <= t) lo = mid; else hi = mid;
      }
      int64_t bw = 0;
      for (int64_t i = 0; i < B; ++i)
        if (excl[i] <= t) bw = i;
      ok = ok && bw == lo && excl[bw] == start[lo] && incl[bw] == start[lo + 1];
    }
    EXPECT(ok, "wave tile lookup differs from the prologue table (B %lld)", (long long)B);
  }
}

// Packed batches of few samples are tiled so that their tile count stays at
// or below two per CU whatever the split of the rows into samples (one tile
// more puts a third equal workgroup on some CU); batches of more samples keep
// four tiles per CU.
static void test_few_sample_tile_bound() {
  uint64_t seed = 777;
  auto next = [&seed]() { seed = seed * 6364136223846793005ull + 1442695040888963407ull; return seed >> 33; };
  for (int cus : {80, 256, 304}) {
    for (int B : {1, 2, 3, 4, 9, 16, 33, 64}) {
      for (int rep = 0; rep < 40; ++rep) {
        std::vector<int64_t> n(B);
        int64_t R = 0;
        for (int b = 0; b < B; ++b) { n[b] = static_cast<int64_t>(next() % (rep % 2 ? 9000 : 700)); R += n[b]; }
        const adaln::WorkspaceLayout w = adaln::bwd_workspace_layout(B, R, 3072, cus, true, 0);
        int64_t tiles = 0;
        for (int b = 0; b < B; ++b) tiles += (n[b] + w.tile_rows - 1) / w.tile_rows;
        const bool ok = tiles <= std::max<int64_t>(2 * cus, B) && tiles <= w.tiles_alloc;
        EXPECT(ok, "few-sample packed batch: %lld tiles on %d CUs (B %d, R %lld, tile_rows %lld)",
               (long long)tiles, cus, B, (long long)R, (long long)w.tile_rows);
      }
    }
  }
  // dense batches: at most two tiles per CU whenever B allows it
  for (int cus : {80, 256, 304})
    for (int64_t B : {1, 2, 3, 5, 6, 7, 8, 100, 511, 600})
      for (int64_t N : {1, 5, 255, 777, 1000, 2000, 3000, 4096, 4097, 18900, 64000}) {
        const adaln::WorkspaceLayout w = adaln::bwd_workspace_layout(B, B * N, 3072, cus, false, N);
        const int64_t tiles = B * ((N + w.tile_rows - 1) / w.tile_rows);
        EXPECT(tiles == w.tiles_max && tiles <= std::max<int64_t>(2 * cus, B),
               "dense batch B %lld N %lld on %d CUs: %lld tiles of %lld rows", (long long)B, (long long)N, cus,
               (long long)tiles, (long long)w.tile_rows);
      }
  EXPECT(adaln::bwd_tiles_per_cu(false, 1000) == 2 && adaln::bwd_tiles_per_cu(true, 64) == 2 &&
             adaln::bwd_tiles_per_cu(true, 65) == 4,
         "tiles per CU: dense 2, packed up to 64 samples 2, more 4");
}

int main() {
  test_offset_clamp();
  test_few_sample_tile_bound();
  test_wave_tile_lookup();
  test_plans();
  test_forward();
  test_forward_varlen();
  test_backward();
  test_backward_varlen();
  test_status_strings();
  std::printf("%d checks, %d failures, %d launches\n", g_checks, g_failures, g_launches);
  return g_failures == 0 ? 0 : 1;
}
