// Internal interface between the host dispatcher (adaln_api.cpp), the host
// planning code (adaln_plan.cpp: row layouts, backward tiling, workspace
// layout) and the kernel launchers (adaln_kernels.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/adaln.h"

namespace adaln {

enum DType : int { F32 = 0, BF16 = 1 };

// How rows are grouped into samples.
//   dense:  sample b owns rows [b*N, (b+1)*N)                 (offsets == nullptr)
//   varlen: sample b owns rows [offsets[b], offsets[b+1])     (device int64 array)
struct RowMap {
  int64_t B;
  int64_t R;
  int64_t N;                 // dense rows per sample (unused for varlen)
  const int64_t* offsets;    // device, B+1 entries, or nullptr for dense
};

// Packed-batch offsets live in device memory and are trusted (the host cannot
// read them without synchronising), so the kernels clamp every offset they
// read into [0, R] and treat a sample whose end lies before its start as
// empty: a malformed table then gives wrong results but no access outside the
// row tensors (constexpr, so the same function serves the kernels and the
// host tests).
constexpr int64_t clamp_row(int64_t v, int64_t R) { return v < 0 ? 0 : (v > R ? R : v); }

// Rows [lo, lo + n) of a packed sample whose offsets are o0 and o1, clamped.
struct RowSpan {
  int64_t lo, n;
};
constexpr RowSpan clamped_span(int64_t o0, int64_t o1, int64_t R) {
  return RowSpan{clamp_row(o0, R), clamp_row(o1, R) > clamp_row(o0, R) ? clamp_row(o1, R) - clamp_row(o0, R) : 0};
}

// Backward tiling: every tile is a run of at most `tile_rows` consecutive rows
// inside one sample.  Sample b's tiles are numbered
// [tile_start(b), tile_start(b+1)).  Dense: tile_start(b) = b * ceil(N/tile_rows).
// Varlen: tile_start lives in the workspace and is written by the prologue.
struct Tiling {
  int64_t tile_rows;
  int64_t tiles_max;         // grid size of the row pass (upper bound for varlen)
  int64_t tiles_alloc;       // tile capacity of the partial-sum buffer (>= any tile count)
  int64_t* tile_start;       // device, B+1 entries (varlen only), else nullptr
  int interleave;            // 1: tile k of a sample takes rows k, k+tiles, ...; 0: contiguous runs
};

// Row layout of the vectorised kernels: a row of D elements is V = D/EPV
// 16-byte vectors; LPR lanes cooperate on a row, each holding VPT vectors
// (vector j*LPR + lane).  NT threads per workgroup form NT/LPR row slots, and
// each slot carries RIF rows per loop iteration.
struct VecPlan {
  bool ok;
  int vpt;
  int lpr;
  int nt;
  int rif;
};

// Largest workgroup of the vectorised kernels: 8 waves, i.e. two per SIMD, so
// the compiler may give each wave up to 256 VGPRs.
constexpr int VEC_MAX_NT = 512;
// Rows each slot handles per loop iteration.  Measured on MI355X, one row
// per slot with more workgroups resident beats deeper per-slot batching or
// register prefetch where a lane holds many elements: both cost VGPRs, hence
// occupancy, which is what keeps HBM requests in flight here.  The forward's
// short rows (at most FWD_RIF2_MAX_VPT vectors per lane) take two rows per
// slot instead: DiT's D = 1152 rows (3 vectors per lane), 8,192 of them, run
// the forward in 8.1 us at two rows per slot and one iteration per workgroup
// against 10.3 us at one row per slot and two iterations.
constexpr int BWD_RIF = 1;
constexpr int FWD_RIF2_MAX_VPT = 3;
// dy + x bytes in flight per CU (its backward tiles, one row each) below
// which a backward workgroup holds two row slots rather than one.
constexpr int64_t BWD_MIN_CU_BYTES = 32768;
constexpr int FWD_MAX_VPT = 8;
constexpr int BWD_MAX_VPT = 4;
// Tile partial sums are stored chunk-major: for each 16-column chunk, the
// tiles' 16-float rows of sum(dy) and sum(dy*xhat) follow each other, so the
// finish reads each chunk's tiles as one contiguous run (on MI355X this cut the
// finish from 10.0 to 6.4 us on the video shape against a tile-major layout).
constexpr int PCOLS = 16;

// Packed batches of at most this many samples are tiled like dense ones (two
// tiles per CU), and the backward kernels rebuild their tile table per wave
// (one sample per lane) instead of reading one written by a prologue launch.
constexpr int64_t PACKED_FEW_SAMPLES = 64;

// Backward tiles per CU: 2 for dense batches and packed batches of few
// samples, 4 for packed batches of more samples.
int bwd_tiles_per_cu(bool varlen, int64_t B);

// Vector plan for the forward (backward = false) or backward kernels; varlen
// and B (samples) select the backward's tiling.
VecPlan plan_vec(int dtype, int64_t D, bool backward, bool varlen = false, int64_t B = 1);

// Dynamic LDS bytes of a vectorised launch with plan p.
size_t vec_lds_bytes(const VecPlan& p, int64_t D, bool backward);

// Launchers.  Each returns hipSuccess or the launch error.  They assume the
// arguments were validated by the caller.
hipError_t launch_fwd(int dtype, const void* x, const void* shift, const void* scale, float eps,
                      const RowMap& rm, int64_t D, bool vec, const VecPlan& vp, int num_cu,
                      hipStream_t stream, void* y, float* mean, float* rstd);

// sums_f32: dscale and dshift are fp32 whatever dtype is (else dtype).
hipError_t launch_bwd(int dtype, const void* dy, const void* x, const void* scale,
                      const float* mean, const float* rstd, const RowMap& rm, int64_t D,
                      bool vec, const VecPlan& vp, const Tiling& tl, float* partial,
                      hipStream_t stream, void* dx, void* dscale, void* dshift, bool sums_f32);

// The two-pass backward: dx rows, then D-tile column partials that read dy
// and x again, then the finish.  Vectorised plans only (vp.ok, 16-byte
// aligned rows).
hipError_t launch_bwd_twopass(int dtype, const void* dy, const void* x, const void* scale,
                              const float* mean, const float* rstd, const RowMap& rm, int64_t D,
                              const VecPlan& vp, const Tiling& tl, float* partial,
                              hipStream_t stream, void* dx, void* dscale, void* dshift);

// Rows per backward tile for R rows in B samples (of N_dense rows each for a
// dense batch) on a device with num_cu compute units.
int64_t bwd_tile_rows(int64_t R, int64_t B, int num_cu, bool varlen, int64_t N_dense);

// Bytes of workspace for the backward (tile table + partial sums).
size_t bwd_workspace_bytes(int64_t B, int64_t R, int64_t D, int num_cu);

// Layout of that workspace.
struct WorkspaceLayout {
  size_t tile_start_off;   // int64 [B+1]
  size_t partial_off;      // fp32 [ceil(D/16)][tiles_alloc][2][16]
  size_t total;
  int64_t tile_rows;
  int64_t tiles_max;
  int64_t tiles_alloc;
};
WorkspaceLayout bwd_workspace_layout(int64_t B, int64_t R, int64_t D, int num_cu, bool varlen,
                                     int64_t N_dense);

// adaln_bwd with the workspace given as a pointer and size (shared by adaln_bwd
// and the no-allocation entry point).
adaln_status_t bwd_dense_with_workspace(const void* dy, const void* x, const void* scale,
                                        const float* mean, const float* rstd, int64_t B, int64_t N,
                                        int64_t D, adaln_dtype_t dtype, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream, void* dx,
                                        void* dscale, void* dshift);

}  // namespace adaln
