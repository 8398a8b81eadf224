"""A float32 model of the kernels' rounding, for the tolerance analysis.

TEST INFRASTRUCTURE ONLY: not the oracle and not the kernels.  It follows
the arithmetic order the HIP kernels use for the quantities whose error
bounds the GPU tests must allow:

* forward statistics of a row laid out as one wave (64 lanes, each holding
  every 64th group of 4 elements): per-lane sequential fp32 sum, mean by
  the product with the rounded reciprocal plus one fma correction, per-lane
  sum of squared deviations with fmas, then a pairwise Chan merge over the
  lanes (adjacent groups, six levels); rstd = 1/sqrt(M2/D + eps);
* the backward's xhat = (x - mean) * rstd, each step rounded to fp32;
* per-tile column partials: a dense sample's rows split over T tiles
  interleaved (tile k takes rows k, k + T, ...), each column summed down its
  tile's rows in row order, sum(dy) with fp32 adds and sum(dy*xhat) with
  fp32 fmas;
* the finish: the tiles' partials added in fp64, one rounding to the output
  type.

Every operation is IEEE round to nearest even in float32; an fma is the
exact product and sum rounded once (computed in float64, where the product
of two float32 values is exact).
"""

from __future__ import annotations

import numpy as np

F = np.float32


def _fma(a, b, c):
    """fp32 fma: a*b + c rounded once (a, b, c float32 arrays)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F)


def lane_layout(D: int) -> np.ndarray:
    """Column indices held by each of 64 lanes, in the order a lane visits
    them: lane l holds 4-element groups l, l + 64, l + 128, ...  D must be a
    multiple of 256."""
    assert D % 256 == 0
    groups = D // 4
    vpt = groups // 64
    idx = np.empty((64, vpt * 4), dtype=np.int64)
    for lane in range(64):
        cols = []
        for j in range(vpt):
            g = lane + 64 * j
            cols += [4 * g + k for k in range(4)]
        idx[lane] = cols
    return idx


def row_stats_f32(x: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """mean and rstd (float32) of each row of x (float32 [R, D]) as the
    one-wave-per-row forward computes them."""
    R, D = x.shape
    idx = lane_layout(D)
    n_lane = idx.shape[1]
    xl = x[:, idx]                                    # [R, 64, n_lane]
    acc = np.zeros((R, 64), dtype=F)
    for k in range(n_lane):
        acc = (acc + xl[:, :, k]).astype(F)
    n = F(n_lane)
    inv_n = F(1.0) / n
    q = (acc * inv_n).astype(F)
    r = _fma(-q, np.full_like(q, n), acc)
    ml = _fma(r, np.full_like(r, inv_n), q)
    sq = np.zeros((R, 64), dtype=F)
    for k in range(n_lane):
        d = (xl[:, :, k] - ml).astype(F)
        sq = _fma(d, d, sq)
    m, s = ml, sq
    cnt = float(n_lane)
    width = 1
    while width < 64:                                 # merge lane groups pairwise
        mo = m.reshape(R, -1, 2)
        so = s.reshape(R, -1, 2)
        ma, mb = mo[:, :, 0], mo[:, :, 1]
        sa, sb = so[:, :, 0], so[:, :, 1]
        dlt = (mb - ma).astype(F)
        half = F(0.5 * cnt)                          # each side covers cnt elements: weight cnt/2
        m = (F(0.5) * (ma + mb).astype(F)).astype(F)
        s = _fma((dlt * dlt).astype(F), np.full_like(dlt, half), (sa + sb).astype(F))
        cnt *= 2
        width *= 2
    mean = m[:, 0]
    var = _fma(s[:, 0], np.full(R, F(1.0) / F(D), dtype=F), np.full(R, F(eps), dtype=F))
    rstd = (F(1.0) / np.sqrt(var).astype(F)).astype(F)
    return mean, rstd


def xhat_f32(x: np.ndarray, mean: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    return ((x - mean[:, None]).astype(F) * rstd[:, None]).astype(F)


def column_sums_f32(dy: np.ndarray, xh: np.ndarray, tiles: int, out_f32: bool = True):
    """dshift and dscale of one dense sample (dy, xh float32 [N, D]) through
    interleaved tiles, fp32 partials, fp64 finish, one final rounding."""
    N, D = dy.shape
    h = np.zeros(D)
    s = np.zeros(D)
    for k in range(tiles):
        rows = np.arange(k, N, tiles)
        ph = np.zeros(D, dtype=F)
        ps = np.zeros(D, dtype=F)
        for r in rows:
            ph = (ph + dy[r]).astype(F)
            ps = _fma(dy[r], xh[r], ps)
        h += ph.astype(np.float64)
        s += ps.astype(np.float64)
    if out_f32:
        return h.astype(F).astype(np.float64), s.astype(F).astype(np.float64)
    return h, s


def dense_tiles(R: int, cus: int = 256) -> int:
    """The dense backward's tile count for R rows on a device with `cus`
    compute units (two tiles per CU, at least 4 rows each)."""
    tile_rows = max(4, -(-R // (2 * cus)))
    return -(-R // tile_rows)
