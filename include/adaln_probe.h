/*
 * adaln_probe.h -- streaming ceiling probes for AMD Instinct MI355X (gfx950).
 *
 * Infrastructure, not part of the operator: these calls measure how fast the
 * device moves bytes in the access mixes of the AdaLN kernels, so that the
 * operator's throughput can be stated against a measured ceiling as well as
 * against the data-sheet HBM peak.  The AdaptiveLoad technical summary
 * (gist.science, paper 2605.17923) motivates the fused kernels by the HBM
 * traffic of the unfused chain (section 1, the memory-wall paragraph, and
 * section 2.B); the forward of the fused operator reads one [R, D] tensor and
 * writes one (the access mix of a copy), its backward row pass reads two and
 * writes one.
 *
 * Every probe streams 16-byte vectors with non-temporal loads and stores over
 * a grid of wg_per_cu 256-thread workgroups per compute unit, each lane
 * keeping `unroll` vectors per operand in flight per loop iteration.
 *
 * Ownership and errors as in adaln.h: device pointers owned by the caller,
 * asynchronous on `stream`, validation before launch, the status code is the
 * only error channel.  Status codes are adaln_status_t from adaln.h.
 */
#ifndef ADALN_PROBE_H_
#define ADALN_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "adaln.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ADALN_PROBE_COPY = 0,       /* out[i] = a[i]: one read, one write (bytes each) */
  ADALN_PROBE_TWO_TO_ONE = 1, /* out[i] = a[i] ^ b[i]: two reads, one write (bytes each) */
  ADALN_PROBE_READ = 2,       /* reads a (bytes); writes adaln_probe_read_out_bytes() bytes to out */
  ADALN_PROBE_WRITE = 3       /* writes out (bytes); reads nothing */
} adaln_probe_mode_t;

/* Largest wg_per_cu accepted. */
#define ADALN_PROBE_MAX_WG_PER_CU 16

/*
 * adaln_probe_stream -- one streaming pass.
 *
 *   mode         one of adaln_probe_mode_t
 *   a, b         device inputs of `bytes` bytes each (b only for TWO_TO_ONE,
 *                a for every mode but WRITE; unused ones may be NULL)
 *   out          device output: `bytes` bytes (COPY, TWO_TO_ONE, WRITE) or
 *                adaln_probe_read_out_bytes(wg_per_cu) bytes (READ)
 *   bytes        a multiple of 16, >= 0
 *   wg_per_cu    1 .. ADALN_PROBE_MAX_WG_PER_CU
 *   unroll       vectors per lane in flight per operand: 1, 2, 4 or 8
 *
 * Every pointer must be 16-byte aligned; buffers must not overlap (not
 * checked).  ADALN_ERR_INVALID_ARG for any violation above; one launch.
 */
adaln_status_t adaln_probe_stream(adaln_probe_mode_t mode, const void* a, const void* b, void* out,
                                  int64_t bytes, int wg_per_cu, int unroll, hipStream_t stream);

/* Bytes a READ probe writes to `out` on the current device (0 if wg_per_cu
 * is out of range or the device cannot be queried). */
size_t adaln_probe_read_out_bytes(int wg_per_cu);

/*
 * Engine-clock probes.  The kernels' rate depends on the engine clock as well
 * as on HBM; these calls record the clock while other work runs (launch them
 * on a second stream beside it).
 *
 * adaln_probe_clock -- one sample, a single wave: it runs `iters` dependent
 * fp32 fmas and writes out[3*slot + 0] = the wall clock when it started,
 * out[3*slot + 1] = shader-clock cycles of the fma chain, out[3*slot + 2] =
 * wall-clock ticks of the chain.  Engine clock over that interval, in kHz:
 * cycles / ticks * adaln_probe_wall_clock_khz().
 *
 *   out      device, 3 * n_slots uint64, 8-byte aligned
 *   slot     0 <= slot < n_slots
 *   iters    1 .. ADALN_PROBE_MAX_CLOCK_ITERS (the length of the fma chain:
 *            a few thousand give samples of a few microseconds)
 *
 * adaln_probe_mark -- a stream-ordered timestamp: out[slot] = the wall clock
 * when the mark runs (after the work enqueued before it on `stream`).
 *   out      device, n_slots uint64, 8-byte aligned; 0 <= slot < n_slots
 *
 * Both: ADALN_ERR_INVALID_ARG for a violation above (nothing launched), one
 * single-wave launch otherwise.
 *
 * adaln_probe_wall_clock_khz -- rate of the wall clock both read, kHz, on
 * the current device (0 if it cannot be queried).
 */
#define ADALN_PROBE_MAX_CLOCK_ITERS (1 << 20)

adaln_status_t adaln_probe_clock(uint64_t* out, int64_t n_slots, int64_t slot, int iters,
                                 hipStream_t stream);
adaln_status_t adaln_probe_mark(uint64_t* out, int64_t n_slots, int64_t slot, hipStream_t stream);
int64_t adaln_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_PROBE_H_ */
