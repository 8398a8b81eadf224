// Streaming ceiling probes for gfx950: how fast this device moves bytes in
// the access mixes of the AdaLN kernels, so their throughput can be judged
// against what the memory system delivers rather than against the data-sheet
// peak alone.  The forward reads one row tensor and writes one (1:1, a
// copy); the backward row pass reads two and writes one (2:1).
//
// Each probe is a grid-stride loop over 16-byte vectors with non-temporal
// accesses (the same `nt` loads and stores the operator's row kernels use),
// a fixed number of vectors per lane in flight per iteration (`unroll`), and
// a grid of `wg_per_cu` 256-thread workgroups per compute unit.  The value
// computed is trivial integer work, so the probes measure the memory system,
// not the ALUs.
//
// The clock probe measures the engine clock itself: one wave times a chain of
// dependent fmas against both the shader-clock cycle counter and the
// constant-rate wall clock, so a stream of such probes beside a workload
// shows the clock the workload ran at, moment by moment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/adaln_probe.h"

#define ADALN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld(const u32x4_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4_t* p, u32x4_t v) { __builtin_nontemporal_store(v, p); }

constexpr int NT = 256;

// MODE: 0 copy (out = a), 1 two-to-one (out = a ^ b), 2 read (xor-reduce a
// into one vector per thread), 3 write (out = a constant pattern).
template <int MODE, int U>
__global__ void __launch_bounds__(NT) stream_kernel(const u32x4_t* __restrict__ a,
                                                    const u32x4_t* __restrict__ b,
                                                    u32x4_t* __restrict__ out, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * NT;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  // full iterations: U vectors per lane, each U*stride-vector chunk in order
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t va[U], vb[U];
    if constexpr (MODE != 3) {
#pragma unroll
      for (int u = 0; u < U; ++u) va[u] = ld(a + i + u * stride);
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int u = 0; u < U; ++u) vb[u] = ld(b + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (MODE == 0) st(out + i + u * stride, va[u]);
      if constexpr (MODE == 1) st(out + i + u * stride, va[u] ^ vb[u]);
      if constexpr (MODE == 2) acc ^= va[u];
      if constexpr (MODE == 3) {
        const u32x4_t p = {static_cast<unsigned>(i + u * stride), 1u, 2u, 3u};
        st(out + i + u * stride, p);
      }
    }
  }
  for (; i < n; i += stride) {           // the ragged tail
    if constexpr (MODE == 0) st(out + i, ld(a + i));
    if constexpr (MODE == 1) st(out + i, ld(a + i) ^ ld(b + i));
    if constexpr (MODE == 2) acc ^= ld(a + i);
    if constexpr (MODE == 3) {
      const u32x4_t p = {static_cast<unsigned>(i), 1u, 2u, 3u};
      st(out + i, p);
    }
  }
  if constexpr (MODE == 2) out[tid] = acc;   // out holds one vector per thread
}

template <int MODE>
hipError_t launch(int unroll, dim3 grid, hipStream_t s, const void* a, const void* b, void* out,
                  int64_t n) {
  const u32x4_t* pa = static_cast<const u32x4_t*>(a);
  const u32x4_t* pb = static_cast<const u32x4_t*>(b);
  u32x4_t* po = static_cast<u32x4_t*>(out);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((stream_kernel<MODE, 1>), grid, dim3(NT), 0, s, pa, pb, po, n); break;
    case 2: hipLaunchKernelGGL((stream_kernel<MODE, 2>), grid, dim3(NT), 0, s, pa, pb, po, n); break;
    case 4: hipLaunchKernelGGL((stream_kernel<MODE, 4>), grid, dim3(NT), 0, s, pa, pb, po, n); break;
    case 8: hipLaunchKernelGGL((stream_kernel<MODE, 8>), grid, dim3(NT), 0, s, pa, pb, po, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One engine-clock sample (a single wave): out[0] = wall clock at the start,
// out[1] = shader-clock cycles of the fma chain, out[2] = its wall-clock ticks.
__global__ void __launch_bounds__(64) clock_kernel(uint64_t* __restrict__ out, int iters) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_readcyclecounter();
  float v = static_cast<float>(threadIdx.x) * 1e-3f;
  for (int i = 0; i < iters; ++i) v = __builtin_fmaf(v, 0.999f, 0.5f);
  asm volatile("" : : "v"(v));             // the chain's result is used
  const uint64_t c1 = __builtin_readcyclecounter();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = r0;
    out[1] = c1 - c0;
    out[2] = r1 - r0;
  }
}

// A stream-ordered timestamp: out[0] = wall clock when the kernel runs.
__global__ void __launch_bounds__(64) mark_kernel(uint64_t* __restrict__ out) {
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) out[0] = r;
}

}  // namespace

ADALN_EXPORT int64_t adaln_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz > 0 ? khz : 0;
}

ADALN_EXPORT adaln_status_t adaln_probe_clock(uint64_t* out, int64_t n_slots, int64_t slot,
                                              int iters, hipStream_t stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 7u)) return ADALN_ERR_INVALID_ARG;
  if (n_slots < 1 || slot < 0 || slot >= n_slots) return ADALN_ERR_INVALID_ARG;
  if (iters < 1 || iters > ADALN_PROBE_MAX_CLOCK_ITERS) return ADALN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, stream, out + 3 * slot, iters);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

ADALN_EXPORT adaln_status_t adaln_probe_mark(uint64_t* out, int64_t n_slots, int64_t slot,
                                             hipStream_t stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 7u)) return ADALN_ERR_INVALID_ARG;
  if (n_slots < 1 || slot < 0 || slot >= n_slots) return ADALN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mark_kernel, dim3(1), dim3(64), 0, stream, out + slot);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

ADALN_EXPORT size_t adaln_probe_read_out_bytes(int wg_per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (wg_per_cu < 1 || wg_per_cu > ADALN_PROBE_MAX_WG_PER_CU || cus <= 0) return 0;
  return static_cast<size_t>(cus) * wg_per_cu * NT * 16;
}

ADALN_EXPORT adaln_status_t adaln_probe_stream(adaln_probe_mode_t mode, const void* a, const void* b,
                                               void* out, int64_t bytes, int wg_per_cu,
                                               int unroll, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0) return ADALN_ERR_INVALID_ARG;
  if (wg_per_cu < 1 || wg_per_cu > ADALN_PROBE_MAX_WG_PER_CU) return ADALN_ERR_INVALID_ARG;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return ADALN_ERR_INVALID_ARG;
  const bool needs_a = mode != ADALN_PROBE_WRITE, needs_b = mode == ADALN_PROBE_TWO_TO_ONE;
  if (mode < ADALN_PROBE_COPY || mode > ADALN_PROBE_WRITE) return ADALN_ERR_INVALID_ARG;
  if (!out || (needs_a && !a) || (needs_b && !b)) return ADALN_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                        reinterpret_cast<uintptr_t>(out);
  if (mis & 15u) return ADALN_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return ADALN_ERR_HIP;
  const int64_t n = bytes / 16;
  if (n == 0) return ADALN_OK;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(cus) * wg_per_cu));
  hipError_t e = hipSuccess;
  switch (mode) {
    case ADALN_PROBE_COPY: e = launch<0>(unroll, grid, stream, a, b, out, n); break;
    case ADALN_PROBE_TWO_TO_ONE: e = launch<1>(unroll, grid, stream, a, b, out, n); break;
    case ADALN_PROBE_READ: e = launch<2>(unroll, grid, stream, a, b, out, n); break;
    case ADALN_PROBE_WRITE: e = launch<3>(unroll, grid, stream, a, b, out, n); break;
  }
  return e == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
