"""Plain fp64 CPU oracle for the fused adaptive-LayerNorm (AdaLN) operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check in the repository's
entry module and the ``cpu_baseline`` leg of the benchmark do.  It shares no
code with the HIP library (no kernels, headers, helpers, tables or constants)
and imports nothing from it.

What it computes
----------------
The AdaptiveLoad technical summary (gist.science, paper 2605.17923), section
2.B "Kernels CUDA Fusionados LayerNorm-Modulate", describes one fused kernel
that performs LayerNorm normalisation and the AdaLN modulation in a single
launch, keeps the per-row mean and variance on chip, and has a backward whose
modulation gradients are column sums over the sequence axis N.  The summary
prints no equation for the operator; the fused kernel collapses an ordinary
chain of framework nodes (same section, "Simplificación de Grafos" bullet), so
its result is that chain's result.  This module writes that chain out in its
plain definition, in float64, with no fusion, blocking or reordering:

  forward  (per token row r of sample b = b(r), D features)
    F1  mean_r   = (1/D) * sum_d x[r,d]
    F2  var_r    = (1/D) * sum_d (x[r,d] - mean_r)^2          (biased, two-pass)
    F3  rstd_r   = 1 / sqrt(var_r + eps)
    F4  xhat     = (x - mean_r) * rstd_r
    F5  y        = xhat * (1 + scale[b]) + shift[b]

  backward (no gradient flows into the saved statistics)
    B1  g        = dy * (1 + scale[b])
    B2  a_r      = (1/D) * sum_d g,   c_r = (1/D) * sum_d g * xhat
    B3  dx       = rstd_r * (g - a_r - xhat * c_r)
    B4  dshift[b,d] = sum over rows r of sample b of dy[r,d]
    B5  dscale[b,d] = sum over rows r of sample b of dy[r,d] * xhat[r,d]

Where the page is silent this module takes the plainest reading: the
modulation multiplies by (1 + scale) and then adds shift (the usual AdaLN
form, so scale = 0 is the identity); LayerNorm has no affine of its own
(scale and shift are the only affine); the variance is the biased one
(divide by D), as LayerNorm defines it; eps is added to the variance inside
the square root; scale and shift are per-sample [B, D] activations broadcast
over the sample's rows; and their gradients are sums over those rows, not
means.  B3 is the derivative of F4 for a row; it is pinned by finite
differences and by torch's fp64 autograd in the oracle tests, not by
retyping.

Rows belong to samples through ``offsets`` (int64, length B+1, non-decreasing,
offsets[0] = 0, offsets[B] = R): sample b owns rows offsets[b] .. offsets[b+1]-1.
A dense [B, N, D] batch is the case offsets[b] = b*N.

It also carries the page's dual-constraint bucket rule (section 2.A), which
sizes the mixed-length workload's buckets.

Parity status: every function here is pinned by tests under ``tests/`` that
do not route through this module's arithmetic (closed forms, invariants,
finite differences, torch fp64 library routines, hand-derived worked
examples).  No function is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16",
    "decode",
    "sample_of_rows",
    "row_stats",
    "adaln_fwd",
    "adaln_bwd",
    "b_shape",
]


# --------------------------------------------------------------------------
# storage decoding (exact): every stored input is widened to float64 before
# any arithmetic.
# --------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE binary32 value, so the
    widening places the pattern in the high half of a 32-bit word.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bf16 bits must be uint16, got {bits.dtype}")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array of dtype 'f32' (float32) or 'bf16' (uint16 bits) -> float64."""
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "f32":
        a = np.asarray(arr)
        if a.dtype != np.float32:
            raise TypeError(f"f32 storage must be float32, got {a.dtype}")
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# row -> sample map
# --------------------------------------------------------------------------
def _check_offsets(offsets: np.ndarray, R: int) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    if off.ndim != 1 or off.size < 2:
        raise ValueError("offsets must be a 1-D array of length B+1 >= 2")
    if off[0] != 0 or off[-1] != R or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0, end at R and never decrease")
    return off


def sample_of_rows(offsets: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Sample index b with offsets[b] <= r < offsets[b+1], for each row r."""
    off = np.asarray(offsets, dtype=np.int64)
    return np.searchsorted(off, np.asarray(rows, dtype=np.int64), side="right") - 1


# --------------------------------------------------------------------------
# forward  (F1 .. F5)
# --------------------------------------------------------------------------
def row_stats(x: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """F1-F3: per-row mean and rstd = 1/sqrt(biased variance + eps), float64.

    The variance is the two-pass form: the mean is taken first, then the
    mean of squared deviations from it.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    mean = x.sum(axis=-1) / D                      # F1
    dev = x - mean[..., None]
    var = (dev * dev).sum(axis=-1) / D             # F2 (divide by D: biased)
    rstd = 1.0 / np.sqrt(var + eps)                # F3 (eps inside the root)
    return mean, rstd


def adaln_fwd(x, shift, scale, eps, offsets, rows=None):
    """AdaLN forward, F1-F5, in float64.

    x       [R, D]  token rows (already decoded to float64)
    shift   [B, D]  per-sample shift
    scale   [B, D]  per-sample scale (the modulation multiplies by 1 + scale)
    eps     float   added to the biased variance inside the square root
    offsets [B+1]   int64 sample boundaries over the R rows
    rows            optional index array: compute only these rows (rows are
                    independent, so this is the same definition restricted)

    Returns (y [len(rows) or R, D], mean [..], rstd [..]) in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    shift = np.asarray(shift, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    R = x.shape[0]
    off = _check_offsets(offsets, R)
    if rows is None:
        rows = np.arange(R, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    xr = x[rows]
    b = sample_of_rows(off, rows)
    mean, rstd = row_stats(xr, eps)                        # F1-F3
    xhat = (xr - mean[:, None]) * rstd[:, None]            # F4
    y = xhat * (1.0 + scale[b]) + shift[b]                 # F5
    return y, mean, rstd


# --------------------------------------------------------------------------
# backward  (B1 .. B5)
# --------------------------------------------------------------------------
def _dx_rows(dy_r, x_r, scale_b, eps):
    """B1-B3 for a block of rows whose modulation rows are scale_b."""
    D = x_r.shape[-1]
    mean, rstd = row_stats(x_r, eps)
    xhat = (x_r - mean[:, None]) * rstd[:, None]
    g = dy_r * (1.0 + scale_b)                             # B1
    a = g.sum(axis=-1) / D                                 # B2
    c = (g * xhat).sum(axis=-1) / D                        # B2
    dx = rstd[:, None] * (g - a[:, None] - xhat * c[:, None])   # B3
    return dx, xhat


def adaln_bwd(dy, x, scale, eps, offsets, rows=None, samples=None):
    """AdaLN backward, B1-B5, in float64.

    dy, x   [R, D]  upstream gradient and the forward input
    scale   [B, D]  per-sample scale
    eps, offsets as in ``adaln_fwd``; the statistics are recomputed here
    rows            optional: dx only for these rows (default all rows)
    samples         optional: dscale/dshift only for these samples
                    (default all samples); each needs all of its rows

    Returns (dx, dscale, dshift); dscale/dshift have one row per requested
    sample.  A sample with no rows has zero sums.
    """
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    R, D = x.shape
    off = _check_offsets(offsets, R)
    B = off.size - 1
    if rows is None:
        rows = np.arange(R, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    b_rows = sample_of_rows(off, rows)
    dx, _ = _dx_rows(dy[rows], x[rows], scale[b_rows], eps)

    if samples is None:
        samples = np.arange(B, dtype=np.int64)
    samples = np.asarray(samples, dtype=np.int64)
    dscale = np.zeros((samples.size, D), dtype=np.float64)
    dshift = np.zeros((samples.size, D), dtype=np.float64)
    for i, b in enumerate(samples):
        lo, hi = int(off[b]), int(off[b + 1])
        if hi == lo:
            continue
        xb = x[lo:hi]
        mean, rstd = row_stats(xb, eps)
        xhat = (xb - mean[:, None]) * rstd[:, None]
        dshift[i] = dy[lo:hi].sum(axis=0)                  # B4
        dscale[i] = (dy[lo:hi] * xhat).sum(axis=0)         # B5
    return dx, dscale, dshift


# --------------------------------------------------------------------------
# dual-constraint bucket size (section 2.A of the same page)
# --------------------------------------------------------------------------
def b_shape(S: int, m_mem: int, m_comp: int, p: float) -> int:
    """Bucket batch size under both constraints of the page's section 2.A.

    The memory constraint caps B*S by m_mem; the polynomial compute
    constraint caps B*S**p by m_comp; the bucket takes the largest B meeting
    both (each bound floored to an integer), but never fewer than one sample.
    """
    if S <= 0:
        raise ValueError("sequence length must be positive")
    by_mem = m_mem // S
    if float(p).is_integer():
        by_comp = m_comp // (S ** int(p))          # exact integer floor
    else:
        by_comp = math.floor(m_comp / (S ** p))
    return max(1, min(by_mem, by_comp))
