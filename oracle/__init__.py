"""fp64 CPU oracle for the AdaLN operator (test infrastructure only).

Only the tests, the repository's smoke check and the benchmark's
``cpu_baseline`` leg may import this package; the product path never does.
"""
from .adaln_ref import (  # noqa: F401
    adaln_bwd,
    adaln_fwd,
    b_shape,
    decode,
    decode_bf16,
    row_stats,
    sample_of_rows,
)
from .sched_ref import cost_model, fit_cost_model, load_cv, plan_groups  # noqa: F401
