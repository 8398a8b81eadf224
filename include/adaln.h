/*
 * adaln.h -- C ABI of the fused adaptive-LayerNorm (AdaLN) library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operator is the fused LayerNorm-modulate of the AdaptiveLoad technical
 * summary (gist.science, paper 2605.17923), section 2.B "Kernels CUDA
 * Fusionados LayerNorm-Modulate": normalisation and modulation in one launch
 * with the row statistics kept on chip (forward bullet), and a backward whose
 * per-sample modulation gradients are sums over the sequence axis N computed
 * with threads pinned to a feature index d so that memory accesses stay
 * contiguous along D (backward bullet, "Reducción Coalescida D-tile").  The
 * summary prints no formula; the operator is the plain chain it fuses:
 *
 *   forward, row r of sample b, D features, fp32 statistics:
 *     mean_r = sum_d x[r,d] / D
 *     rstd_r = 1 / sqrt( sum_d (x[r,d] - mean_r)^2 / D + eps )
 *     xhat   = (x - mean_r) * rstd_r
 *     y      = xhat * (1 + scale[b,:]) + shift[b,:]
 *   backward:
 *     g      = dy * (1 + scale[b,:])
 *     dx     = rstd_r * ( g - mean_d(g) - xhat * mean_d(g * xhat) )
 *     dscale[b,d] = sum over rows of sample b of dy * xhat
 *     dshift[b,d] = sum over rows of sample b of dy
 *
 * Layout.  Every tensor is contiguous and row-major with D innermost:
 * x, y, dy, dx are [R, D] (R token rows; a dense batch is [B, N, D] with
 * R = B*N); shift, scale, dscale, dshift are [B, D]; mean and rstd are fp32
 * [R].  x, y, dy, dx, shift, scale, dscale, dshift all have the element type
 * `dtype` (except the *_f32sums backward entry points, whose dscale and
 * dshift are fp32); statistics and every accumulation are fp32 (the column
 * sums are finished in fp64); every result is rounded to its output type
 * (to nearest, ties to even) once.
 *
 * Ownership.  Every pointer is a device pointer owned by the caller; the
 * library never allocates, frees or synchronises, and keeps no state except
 * a per-device cache of device properties filled on first use (and, for
 * adaln_bwd_noalloc, a static device array and its per-device address).  Every call
 * is enqueued asynchronously on `stream` (NULL = the null stream) and returns
 * as soon as its kernels are enqueued.  Calls on different streams may run
 * concurrently as long as their buffers are disjoint.
 *
 * Errors.  The return code is the only error channel; no exception crosses
 * the ABI.  All arguments are validated before any kernel is enqueued, so a
 * non-OK return from validation means nothing was launched and no output was
 * written.  Only the first failing check is reported.  ADALN_ERR_HIP means a
 * HIP call failed (device query or launch); outputs are then unspecified.
 *
 * Determinism.  For the same inputs, shape, dtype and device, every output is
 * bitwise identical from run to run: every reduction, including the
 * two-stage column reduction behind dscale and dshift, has a fixed order and
 * no floating-point atomics are used.
 *
 * Performance paths.  Rows whose byte length is a multiple of 16 and whose
 * pointers are 16-byte aligned, with D/(elements per 16 bytes) divisible into
 * 16-lane groups, run the vectorised register-resident kernels; every other
 * shape runs a general (slower, equally exact) kernel.  Both meet the same
 * tolerances.
 */
#ifndef ADALN_H_
#define ADALN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds adaln_bwd_f32sums and adaln_bwd_varlen_f32sums; 3: adds adaln_bwd_noalloc */
#define ADALN_ABI_VERSION 3

/* Element type of x, y, dy, dx, shift, scale, dscale, dshift. */
typedef enum {
  ADALN_F32 = 0,  /* IEEE binary32 */
  ADALN_BF16 = 1  /* bfloat16: the upper half of a binary32 */
} adaln_dtype_t;

typedef enum {
  ADALN_OK = 0,
  ADALN_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad eps, bad offsets */
  ADALN_ERR_UNSUPPORTED_DTYPE = 2,  /* dtype is not one of adaln_dtype_t */
  ADALN_ERR_UNSUPPORTED_SHAPE = 3,  /* D above ADALN_MAX_D, or sizes that overflow int64 bytes */
  ADALN_ERR_WORKSPACE_TOO_SMALL = 4,/* backward workspace smaller than adaln_bwd_workspace_size() */
  ADALN_ERR_ALIASING = 5,           /* an output overlaps an input or another output */
  ADALN_ERR_HIP = 6                 /* a HIP runtime call or kernel launch failed */
} adaln_status_t;

/* Largest supported feature dimension. */
#define ADALN_MAX_D 65536

/*
 * adaln_fwd -- forward of a dense batch [B, N, D].
 *
 *   x      [B*N, D]  dtype   input token rows
 *   shift  [B, D]    dtype   per-sample shift
 *   scale  [B, D]    dtype   per-sample scale (rows are multiplied by 1 + scale)
 *   eps              float   added to the biased variance inside the square root;
 *                            finite and >= 0 (with eps = 0 a row of equal values
 *                            has no defined normalisation: its rstd is +inf and
 *                            its y and dx are not finite)
 *   B >= 1, N >= 0, 1 <= D <= ADALN_MAX_D
 *   y      [B*N, D]  dtype   output; must not overlap any input
 *   mean   [B*N]     fp32    saved row means (for adaln_bwd)
 *   rstd   [B*N]     fp32    saved 1/sqrt(var + eps)
 *
 * N == 0 is a valid empty call: nothing is launched.
 * One kernel launch.  Section 2.B, forward bullet.
 */
adaln_status_t adaln_fwd(const void* x, const void* shift, const void* scale, float eps,
                         int64_t B, int64_t N, int64_t D, adaln_dtype_t dtype,
                         hipStream_t stream, void* y, float* mean, float* rstd);

/*
 * adaln_bwd_workspace_size -- infrastructure (no passage of the summary
 * defines it): the storage of section 2.B's two-stage column reduction.
 * Bytes of device workspace every backward entry
 * point (adaln_bwd, adaln_bwd_varlen, their *_f32sums variants and
 * adaln_bwd_twopass) needs for B samples, total_rows rows and D features on
 * the current device.  Returns 0 for invalid sizes.  The size depends on the
 * device's compute-unit count; query it on the device that will run the call.
 */
size_t adaln_bwd_workspace_size(int64_t B, int64_t total_rows, int64_t D, adaln_dtype_t dtype);

/*
 * adaln_bwd -- backward of a dense batch [B, N, D].
 *
 *   dy     [B*N, D]  dtype   upstream gradient of y
 *   x      [B*N, D]  dtype   the forward's input
 *   scale  [B, D]    dtype   the forward's scale
 *   mean, rstd [B*N] fp32    the statistics adaln_fwd saved for this x and eps
 *   B, N, D                  as in adaln_fwd
 *   workspace        device scratch of at least adaln_bwd_workspace_size(B, B*N, D, dtype)
 *                    bytes, 16-byte aligned, owned by the caller; its contents
 *                    on entry are ignored and on exit are unspecified
 *   dx     [B*N, D]  dtype   gradient of x
 *   dscale [B, D]    dtype   gradient of scale: sum over the sample's rows of dy * xhat
 *   dshift [B, D]    dtype   gradient of shift: sum over the sample's rows of dy
 *
 * Outputs must not overlap inputs, each other or the workspace.  With N == 0
 * the call writes zeros to dscale and dshift.  Two launches: a fused row pass
 * (dx plus per-tile column partial sums kept along D) and a deterministic
 * finish that adds each sample's tile partials in fp64 in an order fixed by
 * the shape and the device's CU count, and rounds each sum once.
 * Section 2.B, backward bullet.
 */
adaln_status_t adaln_bwd(const void* dy, const void* x, const void* scale,
                         const float* mean, const float* rstd,
                         int64_t B, int64_t N, int64_t D, adaln_dtype_t dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         void* dx, void* dscale, void* dshift);

/*
 * adaln_fwd_varlen -- forward of B samples packed back to back.
 *
 *   offsets_dev [B+1] int64, DEVICE memory: sample b owns rows
 *                    offsets[b] .. offsets[b+1]-1; offsets[0] = 0,
 *                    offsets[B] = total_rows, non-decreasing.  The host
 *                    cannot read device memory without synchronising, so
 *                    these values are trusted: only B and total_rows are
 *                    validated.
 *   other arguments as in adaln_fwd with R = total_rows >= 0.
 *
 * Samples may have zero rows.  One kernel launch; each row finds its sample
 * by binary search over the offsets.
 *
 * Packed samples of different lengths are the summary's setting: mixed-mode
 * corpora whose sequence lengths range from still images to long videos
 * (section 1, problem statement), batched into groups of equal length and
 * varying batch size by the dual-constraint rule (section 2.A); a packed call
 * runs such a group, or several, in one launch.  The offsets are clamped to
 * [0, total_rows] where the kernels read them, so a malformed table gives
 * wrong results, never an access outside the tensors.
 */
adaln_status_t adaln_fwd_varlen(const void* x, const void* shift, const void* scale, float eps,
                                const int64_t* offsets_dev, int64_t B, int64_t total_rows,
                                int64_t D, adaln_dtype_t dtype, hipStream_t stream,
                                void* y, float* mean, float* rstd);

/*
 * adaln_bwd_varlen -- backward of B packed samples (offsets as in
 * adaln_fwd_varlen: the summary's mixed-length groups, section 1 and section
 * 2.A; the per-sample column sums are section 2.B's backward reduction over N,
 * taken over each sample's own rows).  Three launches: a one-workgroup
 * prologue that turns the offsets into a table of row tiles (each inside one
 * sample) in the workspace, the fused row pass, and the deterministic finish.
 * A sample with zero rows gets zero dscale and dshift.
 */
adaln_status_t adaln_bwd_varlen(const void* dy, const void* x, const void* scale,
                                const float* mean, const float* rstd,
                                const int64_t* offsets_dev, int64_t B, int64_t total_rows,
                                int64_t D, adaln_dtype_t dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                void* dx, void* dscale, void* dshift);

/*
 * adaln_bwd_f32sums, adaln_bwd_varlen_f32sums -- adaln_bwd and
 * adaln_bwd_varlen with dscale and dshift returned in fp32 whatever `dtype`
 * is: the same column sums, rounded once from the fp64 finish to fp32
 * instead of to the I/O type.
 *
 *   dscale [B, D]    fp32    sum over the sample's rows of dy * xhat
 *   dshift [B, D]    fp32    sum over the sample's rows of dy
 *
 * For callers that add these sums to others before rounding: a sequence
 * split over devices, where each device holds the sums over its own rows
 * and the shares are added across devices (the column sums are the only
 * part of the operator that spans rows; section 2.B, backward bullet), or
 * gradient accumulation in fp32 over micro-batches.  dx is
 * bitwise identical to adaln_bwd's / adaln_bwd_varlen's; with dtype ==
 * ADALN_F32 the whole result is.  Every other argument, the workspace (the
 * size adaln_bwd_workspace_size reports), launches and errors as in
 * adaln_bwd / adaln_bwd_varlen; aliasing is checked with dscale and dshift
 * as 4*B*D-byte buffers.
 */
adaln_status_t adaln_bwd_f32sums(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd,
                                 int64_t B, int64_t N, int64_t D, adaln_dtype_t dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 void* dx, float* dscale, float* dshift);

adaln_status_t adaln_bwd_varlen_f32sums(const void* dy, const void* x, const void* scale,
                                        const float* mean, const float* rstd,
                                        const int64_t* offsets_dev, int64_t B,
                                        int64_t total_rows, int64_t D, adaln_dtype_t dtype,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream, void* dx, float* dscale,
                                        float* dshift);

/*
 * adaln_bwd_twopass -- the same backward as adaln_bwd, computed the way the
 * AdaptiveLoad summary lays out its gradient reduction (section 2.B, backward
 * bullet, "Reducción Coalescida D-tile") without fusing it into the dx pass:
 *   1. a row pass that writes dx only;
 *   2. a (n_tile, d_tile) grid that reads dy and x again, each thread pinned
 *      to 8 (bf16) or 4 (fp32) adjacent features of one 16-byte vector,
 *      adding dy and dy * xhat down a contiguous chunk of the sample's rows;
 *   3. the same deterministic finish as adaln_bwd.
 * It moves 2*R*D more elements through HBM than adaln_bwd and exists to
 * measure what the fusion saves.  Arguments, ownership, workspace (the size
 * adaln_bwd_workspace_size reports) and errors as in adaln_bwd, plus:
 * ADALN_ERR_UNSUPPORTED_SHAPE unless dy, x, dx and scale are 16-byte aligned
 * and D fits the vectorised row layout (D*element size a multiple of 16 and
 * the row's 16-byte vectors divisible into 16-lane groups).  dx is bitwise
 * identical to adaln_bwd's; dscale and dshift add the same terms in another
 * fixed order, so they agree with adaln_bwd's to rounding and are bitwise
 * repeatable from run to run.  Three launches.
 */
adaln_status_t adaln_bwd_twopass(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd,
                                 int64_t B, int64_t N, int64_t D, adaln_dtype_t dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 void* dx, void* dscale, void* dshift);

/*
 * adaln_bwd_noalloc -- adaln_bwd without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.
 *
 * The workspace comes from a static device array of the library,
 * ADALN_NOALLOC_SCRATCH_BYTES (32 MiB) on every device the library runs on,
 * held until the process ends; the call itself allocates nothing.  Problems
 * whose adaln_bwd_workspace_size() exceeds it return
 * ADALN_ERR_WORKSPACE_TOO_SMALL before anything is launched (32 MiB holds the
 * workspace of B = 1, N = 64,000, D = 5120 and of 229,368 rows at D = 3072).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device race and give undefined dscale and dshift.  Arguments,
 * outputs, launches, results (bit for bit) and the other errors as in
 * adaln_bwd; ADALN_ERR_HIP also if the array's device address cannot be
 * looked up on first use on a device.
 */
#define ADALN_NOALLOC_SCRATCH_BYTES (32u << 20)

adaln_status_t adaln_bwd_noalloc(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd,
                                 int64_t B, int64_t N, int64_t D, adaln_dtype_t dtype,
                                 hipStream_t stream, void* dx, void* dscale, void* dshift);

/* Infrastructure: human-readable name of a status code (static storage;
 * never NULL; "ADALN_ERR_UNKNOWN" for a value outside adaln_status_t). */
const char* adaln_status_str(adaln_status_t status);

/* Infrastructure: ADALN_ABI_VERSION of the built library, for a caller to
 * check against the header it was compiled with. */
int adaln_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_H_ */
