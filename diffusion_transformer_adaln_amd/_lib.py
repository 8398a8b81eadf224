"""ctypes binding of the C ABI in include/adaln.h (argument marshalling only).

Every function here has the name of the C entry point it wraps.  PyTorch
supplies device memory and the current HIP stream; all computation runs in
the library's HIP kernels.  If the library is not built the import of this
module's functions fails loudly: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libadaln.so")

ADALN_F32 = 0
ADALN_BF16 = 1
ADALN_OK = 0
STATUS_NAMES = {
    0: "ADALN_OK",
    1: "ADALN_ERR_INVALID_ARG",
    2: "ADALN_ERR_UNSUPPORTED_DTYPE",
    3: "ADALN_ERR_UNSUPPORTED_SHAPE",
    4: "ADALN_ERR_WORKSPACE_TOO_SMALL",
    5: "ADALN_ERR_ALIASING",
    6: "ADALN_ERR_HIP",
}

EXPORTED = (
    "adaln_fwd",
    "adaln_bwd",
    "adaln_fwd_varlen",
    "adaln_bwd_varlen",
    "adaln_bwd_twopass",
    "adaln_bwd_f32sums",
    "adaln_bwd_varlen_f32sums",
    "adaln_bwd_workspace_size",
    "adaln_bwd_noalloc",
    "adaln_status_str",
    "adaln_abi_version",
    "adaln_sched_batch_size",
    "adaln_sched_plan",
    "adaln_cost_fit",
    "adaln_load_cv",
    "adaln_probe_stream",
    "adaln_probe_read_out_bytes",
    "adaln_probe_clock",
    "adaln_probe_mark",
    "adaln_probe_wall_clock_khz",
)


class AdaLNError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libadaln.so (once).  torch is imported first so that the library
    binds to the HIP runtime torch already loaded (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m diffusion_transformer_adaln_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    lib.adaln_fwd.argtypes = [_P, _P, _P, ctypes.c_float, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P]
    lib.adaln_fwd.restype = ctypes.c_int
    lib.adaln_fwd_varlen.argtypes = [_P, _P, _P, ctypes.c_float, _P, _I64, _I64, _I64, ctypes.c_int, _P,
                                     _P, _P, _P]
    lib.adaln_fwd_varlen.restype = ctypes.c_int
    lib.adaln_bwd.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, ctypes.c_size_t, _P,
                              _P, _P, _P]
    lib.adaln_bwd.restype = ctypes.c_int
    lib.adaln_bwd_twopass.argtypes = lib.adaln_bwd.argtypes
    lib.adaln_bwd_twopass.restype = ctypes.c_int
    lib.adaln_bwd_f32sums.argtypes = lib.adaln_bwd.argtypes
    lib.adaln_bwd_f32sums.restype = ctypes.c_int
    lib.adaln_bwd_noalloc.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P]
    lib.adaln_bwd_noalloc.restype = ctypes.c_int
    lib.adaln_sched_batch_size.argtypes = [_I64, _I64, _I64, ctypes.c_double]
    lib.adaln_sched_batch_size.restype = _I64
    lib.adaln_sched_plan.argtypes = [_P, _I64, _I64, _I64, ctypes.c_double, _P, _P]
    lib.adaln_sched_plan.restype = ctypes.c_int
    _D = ctypes.POINTER(ctypes.c_double)
    lib.adaln_cost_fit.argtypes = [_P, _P, _P, _I64, ctypes.c_double, ctypes.c_double, _D, _D, _D, _D]
    lib.adaln_cost_fit.restype = ctypes.c_int
    lib.adaln_load_cv.argtypes = [_P, _I64]
    lib.adaln_load_cv.restype = ctypes.c_double
    lib.adaln_bwd_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P,
                                     ctypes.c_size_t, _P, _P, _P, _P]
    lib.adaln_bwd_varlen.restype = ctypes.c_int
    lib.adaln_bwd_varlen_f32sums.argtypes = lib.adaln_bwd_varlen.argtypes
    lib.adaln_bwd_varlen_f32sums.restype = ctypes.c_int
    lib.adaln_bwd_workspace_size.argtypes = [_I64, _I64, _I64, ctypes.c_int]
    lib.adaln_bwd_workspace_size.restype = ctypes.c_size_t
    lib.adaln_status_str.argtypes = [ctypes.c_int]
    lib.adaln_status_str.restype = ctypes.c_char_p
    lib.adaln_abi_version.argtypes = []
    lib.adaln_abi_version.restype = ctypes.c_int
    lib.adaln_probe_stream.argtypes = [ctypes.c_int, _P, _P, _P, _I64, ctypes.c_int, ctypes.c_int, _P]
    lib.adaln_probe_stream.restype = ctypes.c_int
    lib.adaln_probe_read_out_bytes.argtypes = [ctypes.c_int]
    lib.adaln_probe_read_out_bytes.restype = ctypes.c_size_t
    lib.adaln_probe_clock.argtypes = [_P, _I64, _I64, ctypes.c_int, _P]
    lib.adaln_probe_clock.restype = ctypes.c_int
    lib.adaln_probe_mark.argtypes = [_P, _I64, _I64, _P]
    lib.adaln_probe_mark.restype = ctypes.c_int
    lib.adaln_probe_wall_clock_khz.argtypes = []
    lib.adaln_probe_wall_clock_khz.restype = _I64
    _lib = lib
    return lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return ADALN_F32
    if dt == torch.bfloat16:
        return ADALN_BF16
    raise TypeError(f"AdaLN supports float32 and bfloat16, got {dt}")


# The per-call helpers below keep the host cost of a call small (measured on
# MI355X: ~10 us for a forward through the public torch stream and device
# context APIs against ~6 us with these), since the small workloads' kernels
# run for only a few microseconds each.
def _ptr(t):
    return None if t is None else t.data_ptr()


def _expect(t, shape, dtype, name):
    """A tensor the library reads or writes as `shape` elements of `dtype`:
    anything else would make it read or write past the tensor's storage.
    (`shape` is a tuple or torch.Size; the check costs well under a
    microsecond, which matters for the small workloads' per-call cost.)"""
    if t.dtype is not dtype or t.shape != shape:
        if t.shape != shape:
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _expect_stats(t, n, name):
    """mean / rstd: float32 with n elements (any shape, e.g. [B, N] or [R])."""
    if t.dtype is not torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")


def _check_dev(*ts):
    """Index of the one GPU all given tensors live on; they must be contiguous."""
    dev = None
    for t in ts:
        if t is None:
            continue
        i = t.get_device()
        if i < 0:
            raise ValueError("AdaLN tensors must live on a GPU")
        if not t.is_contiguous():
            raise ValueError("AdaLN tensors must be contiguous")
        if dev is None:
            dev = i
        elif i != dev:
            raise ValueError("AdaLN tensors must share one device")
    return dev


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev, stream):
    """Handle of `stream`, else of the current stream of device index `dev`."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _on(dev, fn, *args):
    """Call fn(*args) with device index `dev` current (the library launches on
    the current device)."""
    if torch.cuda.current_device() == dev:
        return fn(*args)
    with torch.cuda.device(dev):
        return fn(*args)


def _raise(fn, st):
    if st != ADALN_OK:
        raise AdaLNError(fn, st)


def _on_stream(stream, made):
    """Tensors allocated here come from the caching allocator's pool of the
    current stream; when the kernels run on another `stream`, record it on
    them so that their memory is not handed out again before that stream's
    work on it is done."""
    if stream is not None:
        for t in made:
            t.record_stream(stream)


# --------------------------------------------------------------------------
# public functions (names of the C entry points)
# --------------------------------------------------------------------------
def adaln_abi_version() -> int:
    return load_library().adaln_abi_version()


def adaln_status_str(status: int) -> str:
    return load_library().adaln_status_str(int(status)).decode()


def adaln_bwd_workspace_size(B: int, total_rows: int, D: int, dtype: torch.dtype, device=None) -> int:
    lib = load_library()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(lib.adaln_bwd_workspace_size(int(B), int(total_rows), int(D), _dtype_code(dtype)))


def adaln_fwd(x, shift, scale, eps: float, y=None, mean=None, rstd=None, stream=None):
    """Forward of a dense batch: x [B, N, D]; shift, scale [B, D].

    Returns (y [B, N, D], mean [B, N] fp32, rstd [B, N] fp32).
    """
    if x.dim() != 3:
        raise ValueError("adaln_fwd expects x of shape [B, N, D]")
    B, N, D = x.shape
    if shift.shape != (B, D) or scale.shape != (B, D):
        raise ValueError("shift and scale must be [B, D]")
    if not (x.dtype == shift.dtype == scale.dtype):
        raise TypeError("x, shift and scale must share a dtype")
    # caller-supplied outputs are checked; the ones made here are right by construction
    made = []
    if y is None:
        y = torch.empty_like(x)
        made.append(y)
    else:
        _expect(y, x.shape, x.dtype, "y")
    if mean is None:
        mean = torch.empty((B, N), dtype=torch.float32, device=x.device)
        made.append(mean)
    else:
        _expect_stats(mean, B * N, "mean")
    if rstd is None:
        rstd = torch.empty((B, N), dtype=torch.float32, device=x.device)
        made.append(rstd)
    else:
        _expect_stats(rstd, B * N, "rstd")
    dev = _check_dev(x, shift, scale, y, mean, rstd)
    _on_stream(stream, made)
    lib = load_library()
    st = _on(dev, lib.adaln_fwd, _ptr(x), _ptr(shift), _ptr(scale), float(eps), B, N, D,
             _dtype_code(x.dtype), _stream(dev, stream), _ptr(y), _ptr(mean), _ptr(rstd))
    _raise("adaln_fwd", st)
    return y, mean, rstd


def adaln_fwd_varlen(x, shift, scale, offsets, eps: float, y=None, mean=None, rstd=None, stream=None):
    """Forward of packed samples: x [R, D]; shift, scale [B, D]; offsets int64 [B+1] on the device."""
    if x.dim() != 2:
        raise ValueError("adaln_fwd_varlen expects x of shape [R, D]")
    R, D = x.shape
    B = shift.shape[0]
    if shift.shape != (B, D) or scale.shape != (B, D) or offsets.shape != (B + 1,):
        raise ValueError("shift/scale must be [B, D] and offsets [B+1]")
    if offsets.dtype != torch.int64:
        raise TypeError("offsets must be int64")
    if not (x.dtype == shift.dtype == scale.dtype):
        raise TypeError("x, shift and scale must share a dtype")
    made = []
    if y is None:
        y = torch.empty_like(x)
        made.append(y)
    else:
        _expect(y, x.shape, x.dtype, "y")
    if mean is None:
        mean = torch.empty((R,), dtype=torch.float32, device=x.device)
        made.append(mean)
    else:
        _expect_stats(mean, R, "mean")
    if rstd is None:
        rstd = torch.empty((R,), dtype=torch.float32, device=x.device)
        made.append(rstd)
    else:
        _expect_stats(rstd, R, "rstd")
    dev = _check_dev(x, shift, scale, offsets, y, mean, rstd)
    _on_stream(stream, made)
    lib = load_library()
    st = _on(dev, lib.adaln_fwd_varlen, _ptr(x), _ptr(shift), _ptr(scale), float(eps), _ptr(offsets),
             B, R, D, _dtype_code(x.dtype), _stream(dev, stream), _ptr(y), _ptr(mean), _ptr(rstd))
    _raise("adaln_fwd_varlen", st)
    return y, mean, rstd


def _workspace(B, R, D, dtype, dev, workspace, made):
    """A caller's workspace (on device index `dev`), else a new one of the
    queried size (appended to `made`)."""
    if workspace is None:
        need = adaln_bwd_workspace_size(B, R, D, dtype, dev)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=torch.device("cuda", dev))
        made.append(workspace)
    elif _check_dev(workspace) != dev:
        raise ValueError("the workspace must be on the tensors' device")
    return workspace, workspace.numel() * workspace.element_size()


def adaln_bwd(dy, x, scale, mean, rstd, workspace=None, dx=None, dscale=None, dshift=None, stream=None):
    """Backward of a dense batch.  Returns (dx [B, N, D], dscale [B, D], dshift [B, D])."""
    return _bwd_dense("adaln_bwd", dy, x, scale, mean, rstd, workspace, dx, dscale, dshift, stream)


def adaln_bwd_f32sums(dy, x, scale, mean, rstd, workspace=None, dx=None, dscale=None, dshift=None,
                      stream=None):
    """adaln_bwd with dscale and dshift in float32 whatever x's dtype (for sums
    that are added to others before rounding)."""
    return _bwd_dense("adaln_bwd_f32sums", dy, x, scale, mean, rstd, workspace, dx, dscale, dshift,
                      stream, torch.float32)


def adaln_bwd_twopass(dy, x, scale, mean, rstd, workspace=None, dx=None, dscale=None, dshift=None,
                      stream=None):
    """The same backward with the column reduction as a separate D-tile pass
    that reads dy and x again (for comparison with the fused adaln_bwd)."""
    return _bwd_dense("adaln_bwd_twopass", dy, x, scale, mean, rstd, workspace, dx, dscale, dshift, stream)


def _bwd_outputs(x, B, D, sums_dtype, dx, dscale, dshift, made):
    """The backward's outputs: the caller's, checked, else new ones (appended
    to `made`)."""
    if dx is None:
        dx = torch.empty_like(x)
        made.append(dx)
    else:
        _expect(dx, x.shape, x.dtype, "dx")
    if dscale is None:
        dscale = torch.empty((B, D), dtype=sums_dtype, device=x.device)
        made.append(dscale)
    else:
        _expect(dscale, (B, D), sums_dtype, "dscale")
    if dshift is None:
        dshift = torch.empty((B, D), dtype=sums_dtype, device=x.device)
        made.append(dshift)
    else:
        _expect(dshift, (B, D), sums_dtype, "dshift")
    return dx, dscale, dshift


def _bwd_dense(fn, dy, x, scale, mean, rstd, workspace, dx, dscale, dshift, stream, sums_dtype=None):
    if x.dim() != 3 or dy.shape != x.shape:
        raise ValueError(f"{fn} expects dy and x of shape [B, N, D]")
    B, N, D = x.shape
    sums_dtype = x.dtype if sums_dtype is None else sums_dtype
    if dy.dtype is not x.dtype:
        raise TypeError(f"dy must be {x.dtype}, got {dy.dtype}")
    _expect(scale, (B, D), x.dtype, "scale")
    _expect_stats(mean, B * N, "mean")
    _expect_stats(rstd, B * N, "rstd")
    made = []
    dx, dscale, dshift = _bwd_outputs(x, B, D, sums_dtype, dx, dscale, dshift, made)
    dev = _check_dev(dy, x, scale, mean, rstd, dx, dscale, dshift)
    lib = load_library()
    workspace, wbytes = _workspace(B, B * N, D, x.dtype, dev, workspace, made)
    _on_stream(stream, made)
    st = _on(dev, getattr(lib, fn), _ptr(dy), _ptr(x), _ptr(scale), _ptr(mean), _ptr(rstd), B, N, D,
             _dtype_code(x.dtype), _ptr(workspace), wbytes, _stream(dev, stream), _ptr(dx),
             _ptr(dscale), _ptr(dshift))
    _raise(fn, st)
    return dx, dscale, dshift


NOALLOC_SCRATCH_BYTES = 32 << 20


def adaln_bwd_noalloc(dy, x, scale, mean, rstd, dx, dscale, dshift, stream=None):
    """adaln_bwd through the entry point that allocates nothing: the outputs
    are the caller's (this wrapper allocates nothing either) and the workspace
    is the library's static device array.  Returns (dx, dscale, dshift)."""
    if x.dim() != 3 or dy.shape != x.shape:
        raise ValueError("adaln_bwd_noalloc expects dy and x of shape [B, N, D]")
    B, N, D = x.shape
    if dy.dtype is not x.dtype:
        raise TypeError(f"dy must be {x.dtype}, got {dy.dtype}")
    _expect(scale, (B, D), x.dtype, "scale")
    _expect_stats(mean, B * N, "mean")
    _expect_stats(rstd, B * N, "rstd")
    _expect(dx, x.shape, x.dtype, "dx")
    _expect(dscale, (B, D), x.dtype, "dscale")
    _expect(dshift, (B, D), x.dtype, "dshift")
    dev = _check_dev(dy, x, scale, mean, rstd, dx, dscale, dshift)
    lib = load_library()
    st = _on(dev, lib.adaln_bwd_noalloc, _ptr(dy), _ptr(x), _ptr(scale), _ptr(mean), _ptr(rstd), B, N, D,
             _dtype_code(x.dtype), _stream(dev, stream), _ptr(dx), _ptr(dscale), _ptr(dshift))
    _raise("adaln_bwd_noalloc", st)
    return dx, dscale, dshift


def adaln_bwd_varlen(dy, x, scale, mean, rstd, offsets, workspace=None, dx=None, dscale=None, dshift=None,
                     stream=None):
    """Backward of packed samples.  Returns (dx [R, D], dscale [B, D], dshift [B, D])."""
    return _bwd_varlen("adaln_bwd_varlen", dy, x, scale, mean, rstd, offsets, workspace, dx, dscale,
                       dshift, stream)


def adaln_bwd_varlen_f32sums(dy, x, scale, mean, rstd, offsets, workspace=None, dx=None, dscale=None,
                             dshift=None, stream=None):
    """adaln_bwd_varlen with dscale and dshift in float32 whatever x's dtype."""
    return _bwd_varlen("adaln_bwd_varlen_f32sums", dy, x, scale, mean, rstd, offsets, workspace, dx,
                       dscale, dshift, stream, torch.float32)


def _bwd_varlen(fn, dy, x, scale, mean, rstd, offsets, workspace, dx, dscale, dshift, stream,
                sums_dtype=None):
    if x.dim() != 2 or dy.shape != x.shape:
        raise ValueError(f"{fn} expects dy and x of shape [R, D]")
    R, D = x.shape
    B = scale.shape[0]
    if offsets.shape != (B + 1,) or offsets.dtype != torch.int64:
        raise ValueError("offsets must be int64 [B+1]")
    sums_dtype = x.dtype if sums_dtype is None else sums_dtype
    if dy.dtype is not x.dtype:
        raise TypeError(f"dy must be {x.dtype}, got {dy.dtype}")
    _expect(scale, (B, D), x.dtype, "scale")
    _expect_stats(mean, R, "mean")
    _expect_stats(rstd, R, "rstd")
    made = []
    dx, dscale, dshift = _bwd_outputs(x, B, D, sums_dtype, dx, dscale, dshift, made)
    dev = _check_dev(dy, x, scale, mean, rstd, offsets, dx, dscale, dshift)
    lib = load_library()
    workspace, wbytes = _workspace(B, R, D, x.dtype, dev, workspace, made)
    _on_stream(stream, made)
    st = _on(dev, getattr(lib, fn), _ptr(dy), _ptr(x), _ptr(scale), _ptr(mean), _ptr(rstd),
             _ptr(offsets), B, R, D, _dtype_code(x.dtype), _ptr(workspace), wbytes,
             _stream(dev, stream), _ptr(dx), _ptr(dscale), _ptr(dshift))
    _raise(fn, st)
    return dx, dscale, dshift


# ---------------------------------------------------------------------------
# host-side scheduling (include/adaln_sched.h); numpy arrays in, no device use
# ---------------------------------------------------------------------------
def _host(a, dtype):
    import numpy as np

    return np.ascontiguousarray(a, dtype=dtype)


def adaln_sched_batch_size(S: int, m_mem: int, m_comp: int, p: float) -> int:
    """B_shape(S) = max(1, min(m_mem // S, floor(m_comp / S**p))); raises on bad arguments."""
    v = load_library().adaln_sched_batch_size(int(S), int(m_mem), int(m_comp), float(p))
    if v < 0:
        raise AdaLNError("adaln_sched_batch_size", 1)
    return int(v)


def adaln_sched_plan(lengths, m_mem: int, m_comp: int, p: float):
    """Group index of every sample (int64 numpy array) and the group count."""
    import numpy as np

    lengths = _host(lengths, np.int64)
    group_of = np.empty(lengths.size, dtype=np.int64)
    n_groups = ctypes.c_int64(0)
    st = load_library().adaln_sched_plan(lengths.ctypes.data if lengths.size else None, lengths.size, int(m_mem),
                                         int(m_comp), float(p), group_of.ctypes.data if lengths.size else None,
                                         ctypes.addressof(n_groups))
    _raise("adaln_sched_plan", st)
    return group_of, int(n_groups.value)


def adaln_cost_fit(B, S, t, p_lo: float = 0.5, p_hi: float = 4.0):
    """Least-squares fit of t = a + b*B*S**p; returns (a, b, p, rss)."""
    import numpy as np

    B, S, t = _host(B, np.float64), _host(S, np.float64), _host(t, np.float64)
    if not (B.size == S.size == t.size):
        raise ValueError("B, S and t must have the same length")
    out = [ctypes.c_double(0.0) for _ in range(4)]
    st = load_library().adaln_cost_fit(B.ctypes.data, S.ctypes.data, t.ctypes.data, B.size, float(p_lo),
                                       float(p_hi), *[ctypes.byref(o) for o in out])
    _raise("adaln_cost_fit", st)
    return tuple(o.value for o in out)


def adaln_load_cv(loads) -> float:
    """Coefficient of variation (population std / mean) of per-worker loads."""
    import numpy as np

    x = _host(loads, np.float64)
    return float(load_library().adaln_load_cv(x.ctypes.data if x.size else None, x.size))


# ---------------------------------------------------------------------------
# streaming ceiling probes (include/adaln_probe.h)
# ---------------------------------------------------------------------------
PROBE_MODES = {"copy": 0, "two_to_one": 1, "read": 2, "write": 3}


def adaln_probe_read_out_bytes(wg_per_cu: int, device=None) -> int:
    lib = load_library()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(lib.adaln_probe_read_out_bytes(int(wg_per_cu)))


def adaln_probe_stream(mode: str, a, b, out, wg_per_cu: int, unroll: int, nbytes=None, stream=None):
    """One streaming pass over uint8 (or any) device tensors: `mode` is one of
    PROBE_MODES; nbytes defaults to the byte size of `out` (copy, two_to_one,
    write) or of `a` (read).  Sizes are checked here, since the library cannot
    see buffer extents."""
    code = PROBE_MODES[mode]
    nb = lambda t: t.numel() * t.element_size()
    if nbytes is None:
        nbytes = nb(a) if mode == "read" else nb(out)
    for t, need in ((a, mode != "write"), (b, mode == "two_to_one")):
        if need and (t is None or nb(t) < nbytes):
            raise ValueError(f"probe input smaller than {nbytes} bytes")
    dev = _check_dev(a, b, out)
    if mode == "read":
        if nb(out) < adaln_probe_read_out_bytes(wg_per_cu, dev):
            raise ValueError("read probe output too small")
    elif nb(out) < nbytes:
        raise ValueError(f"probe output smaller than {nbytes} bytes")
    lib = load_library()
    st = _on(dev, lib.adaln_probe_stream, code, _ptr(a), _ptr(b), _ptr(out), int(nbytes), int(wg_per_cu),
             int(unroll), _stream(dev, stream))
    _raise("adaln_probe_stream", st)


def _slots(out, per):
    """Slots of an int64 device tensor holding `per` uint64 values each."""
    if out.dtype != torch.int64 or not out.is_contiguous() or out.numel() < per:
        raise ValueError("probe output must be a contiguous int64 tensor")
    return out.numel() // per


def adaln_probe_clock(out, slot: int, iters: int, stream=None):
    """One engine-clock sample into out[3*slot : 3*slot+3] (int64 device
    tensor): wall clock at the start, shader-clock cycles, wall-clock ticks."""
    dev = _check_dev(out)
    lib = load_library()
    st = _on(dev, lib.adaln_probe_clock, _ptr(out), _slots(out, 3), int(slot), int(iters), _stream(dev, stream))
    _raise("adaln_probe_clock", st)


def adaln_probe_mark(out, slot: int, stream=None):
    """Stream-ordered timestamp into out[slot] (int64 device tensor)."""
    dev = _check_dev(out)
    lib = load_library()
    st = _on(dev, lib.adaln_probe_mark, _ptr(out), _slots(out, 1), int(slot), _stream(dev, stream))
    _raise("adaln_probe_mark", st)


def adaln_probe_wall_clock_khz(device=None) -> int:
    """Rate of the wall clock the clock probes read, kHz (0 if unknown)."""
    lib = load_library()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(lib.adaln_probe_wall_clock_khz())
