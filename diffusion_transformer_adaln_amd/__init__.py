"""Fused AdaLN (LayerNorm + per-sample modulation) for AMD MI355X (gfx950).

The operator runs in hand-written HIP kernels behind the C ABI declared in
include/adaln.h; this package holds those sources (csrc/), the build step and
a ctypes binding whose functions carry the C entry points' names.  The same
library carries the host-side batch scheduler of include/adaln_sched.h and
the streaming ceiling and engine-clock probes of include/adaln_probe.h.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    AdaLNError,
    adaln_abi_version,
    adaln_bwd,
    adaln_bwd_f32sums,
    adaln_bwd_noalloc,
    adaln_bwd_twopass,
    adaln_bwd_varlen,
    adaln_bwd_varlen_f32sums,
    adaln_bwd_workspace_size,
    adaln_cost_fit,
    adaln_fwd,
    adaln_fwd_varlen,
    adaln_load_cv,
    adaln_probe_clock,
    adaln_probe_mark,
    adaln_probe_read_out_bytes,
    adaln_probe_stream,
    adaln_probe_wall_clock_khz,
    adaln_sched_batch_size,
    adaln_sched_plan,
    adaln_status_str,
    load_library,
)
