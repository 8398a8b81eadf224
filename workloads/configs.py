"""Seeded synthetic inputs for the AdaLN workloads.

This module only draws numbers and lays them out; it holds none of the
operator's arithmetic.  Both the HIP path (through the tests and the
benchmark) and the fp64 oracle consume what it produces, so it imports
neither of them.

Workloads (shapes and value distributions of the DiT / MMDiT / video-DiT
training described on the AdaptiveLoad summary page, which trains Wan 2.1 on
a mixed image/video corpus; none of that corpus is reproduced: the arrays
below are seeded Gaussian stand-ins of the same shapes):

  tiny_fp32    B=1, N=256,  D=128,  fp32; x = z + o_r, z~N(0,1), per-row o_r~N(0,2);
               dy~N(0,1)
  dit_bf16     B=8, N=1024, D=1152, bf16; x~N(0,1); dy~N(0,1e-2)
  mmdit_bf16   two streams, D=3072, bf16: text B=2,N=512 and image B=2,N=4096;
               x~N(0,1) with 1% of each stream's rows multiplied by 20;
               dy~N(0,1e-2); each stream has its own shift/scale
  video_bf16   B=1, N=18900, D=5120, bf16; x~N(0,1); dy~N(0,1e-3)
  mmdit_packed_bf16  the two MMDiT streams' data as one packed batch of four
               samples (512, 512, 4096, 4096 rows), one call per direction
  ragged_bf16  D=3072, bf16, packed rows of 277 samples: 256 samples of 256
               rows, 16 of 4096, 4 of 16384, 1 of 32760 (bucket sizes from the
               page's dual-constraint rule with M_mem=65536, M_comp=2^30, p=2);
               x~N(0,1); dy~N(0,1e-2)

Everywhere shift and scale are drawn per (sample, feature) from N(0, 0.1) and
eps is 1e-6.  N(0, s) means standard deviation s.

Random streams: each tensor has its own child of ``SeedSequence(seed)``
(x, row extras, shift, scale, dy), and large tensors are drawn in fixed
chunks, each chunk from its own grandchild stream, so the bits depend only on
the seed and the shape, never on how many threads drew them.  Values are
drawn as float32 and stored either as float32 or as bfloat16 bit patterns
(uint16) rounded to nearest, ties to even.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# elements drawn per child stream; fixed so the bits never depend on threading
_CHUNK = 1 << 22

EPS = 1e-6
MOD_SIGMA = 0.1

# Mixed-length workload: (sequence length, samples in its bucket).  The
# sample counts are the dual-constraint bucket sizes for M_mem=65536,
# M_comp=2^30, p=2; the oracle tests recompute them from the page's rule.
RAGGED_BUCKETS = ((256, 256), (4096, 16), (16384, 4), (32760, 1))
RAGGED_D = 3072


@dataclass(frozen=True)
class Problem:
    """One AdaLN call: shapes, storage dtype and value distributions."""

    name: str
    dtype: str                      # "f32" or "bf16"
    D: int
    lengths: tuple                  # rows per sample, N_b
    dense: bool                     # all N_b equal and called through the dense entry points
    dy_sigma: float
    eps: float = EPS
    row_offset_sigma: float = 0.0   # per-row scalar offset added to x (tiny config)
    outlier_frac: float = 0.0       # fraction of rows multiplied by outlier_gain
    outlier_gain: float = 20.0
    mod_sigma: float = MOD_SIGMA

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def R(self) -> int:
        return int(sum(self.lengths))

    @property
    def N(self) -> int:
        """Rows per sample for a dense problem."""
        if not self.dense:
            raise ValueError(f"{self.name} is not dense")
        return int(self.lengths[0]) if self.lengths else 0

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclass
class ProblemData:
    problem: Problem
    x: np.ndarray          # [R, D] float32 or uint16 (bf16 bits)
    shift: np.ndarray      # [B, D]
    scale: np.ndarray      # [B, D]
    dy: np.ndarray         # [R, D]
    offsets: np.ndarray    # [B+1] int64
    meta: dict = field(default_factory=dict)


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------
def ragged_lengths(shuffle_seed: int | None = None) -> tuple:
    lens = []
    for S, count in RAGGED_BUCKETS:
        lens += [S] * count
    if shuffle_seed is not None:
        perm = np.random.Generator(np.random.PCG64(shuffle_seed)).permutation(len(lens))
        lens = [lens[i] for i in perm]
    return tuple(lens)


CONFIGS = {
    "tiny_fp32": (
        Problem("tiny_fp32", "f32", 128, (256,), True, dy_sigma=1.0, row_offset_sigma=2.0),
    ),
    "dit_bf16": (
        Problem("dit_bf16", "bf16", 1152, (1024,) * 8, True, dy_sigma=1e-2),
    ),
    "mmdit_bf16": (
        Problem("mmdit_text_bf16", "bf16", 3072, (512,) * 2, True, dy_sigma=1e-2, outlier_frac=0.01),
        Problem("mmdit_image_bf16", "bf16", 3072, (4096,) * 2, True, dy_sigma=1e-2, outlier_frac=0.01),
    ),
    "video_bf16": (
        Problem("video_bf16", "bf16", 5120, (18900,), True, dy_sigma=1e-3),
    ),
    "ragged_bf16": (
        Problem("ragged_bf16", "bf16", RAGGED_D, ragged_lengths(), False, dy_sigma=1e-2),
    ),
    # the sequence length at which the AdaptiveLoad summary quotes its backward
    # speed-up and activation saving (section 4, kernel and memory bullets)
    "long64k_bf16": (
        Problem("long64k_bf16", "bf16", 5120, (64000,), True, dy_sigma=1e-3),
    ),
}

CONFIG_SEEDS = {"tiny_fp32": 1, "dit_bf16": 2, "mmdit_bf16": 3, "video_bf16": 4, "ragged_bf16": 5,
                "long64k_bf16": 6}

# Workloads made by packing another workload's problems back to back into one
# packed batch (same drawn data, one call per direction instead of one per
# problem): the MMDiT text and image streams as four samples of 512, 512,
# 4096 and 4096 rows, each with its own modulation.
PACKED_CONFIGS = {"mmdit_packed_bf16": "mmdit_bf16"}


# --------------------------------------------------------------------------
# encoding
# --------------------------------------------------------------------------
def encode_bf16_rne(f: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN with the same sign.
    """
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def _store(f32: np.ndarray, dtype: str) -> np.ndarray:
    return encode_bf16_rne(f32) if dtype == "bf16" else np.ascontiguousarray(f32, dtype=np.float32)


# --------------------------------------------------------------------------
# chunked seeded draws
# --------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_f32(ss: np.random.SeedSequence, n: int, sigma: float) -> np.ndarray:
    """n float32 draws of N(0, sigma), in fixed chunks of independent streams."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks == 0:
        return out
    children = ss.spawn(nchunks)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if sigma != 1.0:
            out[lo:hi] *= np.float32(sigma)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _encode_chunked(f32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype != "bf16" or f32.size <= _CHUNK:
        return _store(f32, dtype)
    flat = f32.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    nchunks = (flat.size + _CHUNK - 1) // _CHUNK

    def enc(i):
        lo, hi = i * _CHUNK, min(flat.size, (i + 1) * _CHUNK)
        out[lo:hi] = encode_bf16_rne(flat[lo:hi])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(enc, range(nchunks)))
    return out.reshape(f32.shape)


def make_problem_data(problem: Problem, seed: int) -> ProblemData:
    """Draw one problem's inputs from ``seed`` (see the module docstring)."""
    R, D, B = problem.R, problem.D, problem.B
    ss = np.random.SeedSequence(seed)
    s_x, s_extra, s_shift, s_scale, s_dy = ss.spawn(5)

    x = _normal_f32(s_x, R * D, 1.0).reshape(R, D)
    g_extra = np.random.Generator(np.random.PCG64(s_extra))
    meta = {}
    if problem.row_offset_sigma:
        o = g_extra.standard_normal(R, dtype=np.float32) * np.float32(problem.row_offset_sigma)
        x += o[:, None]
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(problem.lengths, dtype=np.int64))
    if problem.outlier_frac:
        k = int(round(problem.outlier_frac * R))
        rows = np.sort(g_extra.choice(R, size=k, replace=False)) if k else np.zeros(0, np.int64)
        x[rows] *= np.float32(problem.outlier_gain)
        meta["outlier_rows"] = rows
    shift = _normal_f32(s_shift, B * D, problem.mod_sigma).reshape(B, D)
    scale = _normal_f32(s_scale, B * D, problem.mod_sigma).reshape(B, D)
    dy = _normal_f32(s_dy, R * D, problem.dy_sigma).reshape(R, D)

    dt = problem.dtype
    return ProblemData(
        problem=problem,
        x=_encode_chunked(x, dt),
        shift=_store(shift, dt),
        scale=_store(scale, dt),
        dy=_encode_chunked(dy, dt),
        offsets=offsets,
        meta=meta,
    )


def pack(pds: list, name: str) -> ProblemData:
    """Several problems' data (same D and dtype) as one packed batch: their
    samples in order, rows concatenated, each sample keeping its modulation."""
    p0 = pds[0].problem
    assert all(pd.problem.D == p0.D and pd.problem.dtype == p0.dtype for pd in pds)
    lengths = tuple(n for pd in pds for n in pd.problem.lengths)
    problem = Problem(name, p0.dtype, p0.D, lengths, False, dy_sigma=p0.dy_sigma, eps=p0.eps,
                      outlier_frac=p0.outlier_frac, outlier_gain=p0.outlier_gain, mod_sigma=p0.mod_sigma)
    offsets = np.zeros(len(lengths) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    cat = lambda k: np.concatenate([getattr(pd, k) for pd in pds], axis=0)
    return ProblemData(problem=problem, x=cat("x"), shift=cat("shift"), scale=cat("scale"), dy=cat("dy"),
                       offsets=offsets, meta={"packed_from": [pd.problem.name for pd in pds]})


def config_names() -> list:
    return list(CONFIGS) + list(PACKED_CONFIGS)


def make_config(name: str, seed: int | None = None) -> list:
    """All problems of a named workload, each with its own derived seed."""
    if name in PACKED_CONFIGS:
        return [pack(make_config(PACKED_CONFIGS[name], seed), name)]
    base = CONFIG_SEEDS[name] if seed is None else seed
    return [make_problem_data(p, base * 1000 + i) for i, p in enumerate(CONFIGS[name])]


def custom_problem(dtype: str, D: int, lengths, dense: bool | None = None, dy_sigma: float = 1e-2,
                   eps: float = EPS, outlier_frac: float = 0.0, row_offset_sigma: float = 0.0,
                   name: str = "custom") -> Problem:
    lengths = tuple(int(n) for n in lengths)
    if dense is None:
        dense = len(set(lengths)) <= 1
    return Problem(name, dtype, int(D), lengths, dense, dy_sigma=dy_sigma, eps=eps,
                   outlier_frac=outlier_frac, row_offset_sigma=row_offset_sigma)


def algorithmic_bytes(problem: Problem) -> dict:
    """Minimal HBM traffic of one forward and one backward call.

    forward:  read x, write y (R*D elements each), write mean and rstd
              (fp32, 8 bytes per row), read shift and scale (B*D each).
    backward: read dy and x, write dx (R*D each), read mean and rstd, read
              scale, write dscale and dshift (B*D each).
    Workspace traffic is excluded: it is overhead, not part of the method.
    """
    R, D, B, s = problem.R, problem.D, problem.B, problem.esize
    fwd = 2 * R * D * s + 8 * R + 2 * B * D * s
    bwd = 3 * R * D * s + 8 * R + 3 * B * D * s
    return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}
