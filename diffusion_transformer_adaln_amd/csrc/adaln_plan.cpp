// Host planning for the AdaLN kernels: the vectorised row layout, the
// backward's tiling and the layout of its workspace.  Plain C++ (no device
// code), shared by the dispatcher and the kernel launchers, and compiled on
// its own by the host validation test.

#include <stddef.h>
#include <stdint.h>

#include "adaln_internal.hpp"

namespace adaln {

// Dynamic LDS of a vectorised launch: double-buffered per-row reduction
// partials, plus the [slots][D] slot-combine buffer of a multi-slot backward.
size_t vec_lds_bytes(const VecPlan& p, int64_t D, bool backward) {
  const int nslots = p.nt / p.lpr;
  const int unit = (p.lpr % 64 == 0) ? 64 : (p.lpr == 32 ? 32 : 16);
  const int groups = p.lpr / unit;
  const int rif = p.rif;
  size_t b = groups > 1 || backward ? 2 * static_cast<size_t>(nslots) * rif * groups * 2 * sizeof(float) : 0;
  if (backward && nslots > 1) b += static_cast<size_t>(nslots) * D * sizeof(float);
  return b;
}

// Backward tiles per compute unit for dense batches: a tile's column partials
// cost 8*D bytes written and read again, so fewer, longer tiles are cheaper,
// but a CU needs enough rows in flight.  Two per CU measured best (backward
// call, video shape: one 147 us, two 102, three 128, four 142; MMDiT 42.9,
// 37.9, 42.8, 44.1; DiT 24.2, 20.9, 26.1, 24.7).
constexpr int BWD_TILES_PER_CU = 2;
// Packed batches of many samples (more than PACKED_FEW_SAMPLES) mix short and
// long samples, so their tiles vary in length; four tiles per CU lets the
// workgroup dispatcher even out the load (mixed 256..32760-row samples at
// D = 3072, backward call: 946 us at two per CU, 914 at three, 862 at four,
// 899 at six, 872 at eight).  Packed batches of few samples are tiled like
// dense ones (two per CU, see bwd_tile_rows).
constexpr int BWD_VARLEN_TILES_PER_CU = 4;

int bwd_tiles_per_cu(bool varlen, int64_t B) {
  return varlen && B > PACKED_FEW_SAMPLES ? BWD_VARLEN_TILES_PER_CU : BWD_TILES_PER_CU;
}

// Row layout for a D-wide row: VPT vectors per lane over LPR = V/VPT lanes,
// LPR a multiple of 16.  Measured on MI355X (video shape, D = 5120 bf16):
//   forward  about 40 elements per lane (two waves per row at D = 5120) with
//            two rows per workgroup is fastest; one wave per row runs out of
//            registers, and wide rows of 8-16 elements per lane spend their
//            time in cross-wave reductions;
//   backward 16 elements per lane (VPT = 2) keeps the per-column
//            accumulators, the modulation row and the row data small enough
//            for four waves per SIMD.
// Ties prefer rows that cover whole waves (no partial-wave reductions).
VecPlan plan_vec(int dtype, int64_t D, bool backward, bool varlen, int64_t B) {
  VecPlan best{false, 0, 0, 0, 1};
  const int max_vpt = backward ? BWD_MAX_VPT : FWD_MAX_VPT;
  const int epv = dtype == BF16 ? 8 : 4;
  if (D <= 0 || D % epv != 0) return best;
  const int64_t V = D / epv;
  const int want = backward ? 16 : 40;           // elements per lane
  int best_score = 1 << 30;
  for (int vpt = 1; vpt <= max_vpt; ++vpt) {
    if (V % vpt) continue;
    const int64_t lpr = V / vpt;
    if (lpr % 16 || lpr > VEC_MAX_NT) continue;
    const int rif = backward ? BWD_RIF : (vpt <= FWD_RIF2_MAX_VPT ? 2 : 1);
    VecPlan p{true, vpt, static_cast<int>(lpr), 0, rif};
    // threads per workgroup: a multiple of both the row lanes and the wave,
    // at least 128 (short rows share a workgroup)
    int nt = p.lpr;
    while (nt % 64) nt += p.lpr;
    const int min_nt = 128;
    while (nt < min_nt && nt * 2 <= VEC_MAX_NT) nt *= 2;
    if (nt > VEC_MAX_NT) continue;
    // backward: a workgroup of one row slot takes a second slot when the
    // CU's tiles, one row each, would hold less than BWD_MIN_CU_BYTES of dy
    // and x in flight.  Dense D = 3072 bf16 (two tiles of 12 KB rows): MMDiT's
    // 8,192-row image stream 42.6 -> 38.0 us per backward, its 1,024-row text
    // stream 17.9 -> 15.1 us with 4-row tiles (below); packed batches of few
    // samples take the same rule.  Packed batches of many samples at
    // D = 3072 (four tiles, 48 KB) were 3% slower with two slots; dense
    // D = 5120 (40 KB) too.
    const int64_t esize = dtype == BF16 ? 2 : 4;
    const int64_t tiles_per_cu = bwd_tiles_per_cu(varlen, B);
    if (backward && nt == p.lpr && tiles_per_cu * 2 * D * esize < BWD_MIN_CU_BYTES &&
        2 * nt <= VEC_MAX_NT)
      nt *= 2;
    p.nt = nt;
    if (vec_lds_bytes(p, D, backward) > 65536) continue;
    const int el = vpt * epv;
    const int score = (el > want ? el - want : want - el) + (lpr % 64 ? 16 : 0);
    if (score < best_score) { best_score = score; best = p; }
  }
  return best;
}

// Short batches: tiles of at least BWD_MIN_TILE_ROWS rows, so the partial
// sums (8*D bytes a tile) stay below the rows' own bytes and each workgroup
// keeps several rows in flight (MMDiT's 1,024-row text stream at D = 3072:
// 15.1 us per backward with 4-row tiles, 18.3 with 2, 16.4 with 8).
constexpr int64_t BWD_MIN_TILE_ROWS = 4;
//
// A packed batch of few samples ends each sample in a partial tile, so it has
// up to B tiles more than R / tile_rows; its tiles are sized for target - B
// of them, which keeps the count at or below target (two per CU).  One tile
// too many puts a third equal workgroup on some CU, which then finishes last:
// four packed samples of D = 3072 summing to 9,216 rows, fwd+bwd step 80.1 us
// with 514 tiles of 18 rows against 67.0 us for a split into exactly 512, and
// 67.5 us with the tiles sized this way (73.1 at four tiles per CU; the
// one-sample 18,900-row batch at D = 5120: 173.9 against 199.8 us).
//
// A dense batch of B samples of N rows has B * ceil(N / tile_rows) tiles,
// which can exceed the target by up to B - 1 (B = 3, N = 4096: 513 tiles of
// 24 rows); its tiles are lengthened until at most target / B fit in a
// sample, which leaves every batch that already fits as it was.
int64_t bwd_tile_rows(int64_t R, int64_t B, int num_cu, bool varlen, int64_t N_dense) {
  const int64_t target = static_cast<int64_t>(num_cu) * bwd_tiles_per_cu(varlen, B);
  const int64_t slots = varlen && B <= PACKED_FEW_SAMPLES && target > B ? target - B : target;
  int64_t rows = R <= 0 ? 1 : (R + slots - 1) / slots;
  if (!varlen && N_dense > 0 && B > 0 && target / B >= 1) {
    const int64_t per_sample = target / B;
    const int64_t fit = (N_dense + per_sample - 1) / per_sample;
    if (fit > rows) rows = fit;
  }
  return rows < BWD_MIN_TILE_ROWS ? BWD_MIN_TILE_ROWS : rows;
}

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

WorkspaceLayout bwd_workspace_layout(int64_t B, int64_t R, int64_t D, int num_cu, bool varlen,
                                     int64_t N_dense) {
  WorkspaceLayout w{};
  w.tile_rows = bwd_tile_rows(R, B, num_cu, varlen, N_dense);
  const int64_t bound = (R + w.tile_rows - 1) / w.tile_rows + B;   // tiles of any row split
  w.tiles_alloc = bound;
  w.tiles_max = varlen ? bound : B * ((N_dense + w.tile_rows - 1) / w.tile_rows);
  w.tile_start_off = 0;
  w.partial_off = align256(static_cast<size_t>(B + 1) * sizeof(int64_t));
  const int64_t chunks = (D + PCOLS - 1) / PCOLS;
  w.total = w.partial_off +
            static_cast<size_t>(chunks) * static_cast<size_t>(bound) * 2 * PCOLS * sizeof(float);
  return w;
}

// Enough for either entry point: the packed layout's tile bound covers any
// row split, and the dense one is checked as well in case its tiles are finer.
size_t bwd_workspace_bytes(int64_t B, int64_t R, int64_t D, int num_cu) {
  const size_t packed = bwd_workspace_layout(B, R, D, num_cu, true, 0).total;
  const size_t dense = bwd_workspace_layout(B, R, D, num_cu, false, B > 0 ? R / B : 0).total;
  return packed > dense ? packed : dense;
}

}  // namespace adaln
