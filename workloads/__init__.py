"""Seeded synthetic workloads for AdaLN (no operator arithmetic here)."""
from .configs import (  # noqa: F401
    CONFIG_SEEDS,
    CONFIGS,
    PACKED_CONFIGS,
    RAGGED_BUCKETS,
    RAGGED_D,
    Problem,
    ProblemData,
    algorithmic_bytes,
    config_names,
    custom_problem,
    encode_bf16_rne,
    make_config,
    make_problem_data,
    pack,
    ragged_lengths,
)
