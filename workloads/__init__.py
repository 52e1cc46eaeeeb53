"""Seeded synthetic workloads for sparse bidirectional attention.

This package holds the workload descriptions (shapes, step schedules and
budgets, as plain parameters) and the seeded input generator.  It is the one
module shared by the GPU library's tests and benchmark and by the fp64 oracle;
it contains none of the attention or selection arithmetic of the method.
"""

from .configs import LOSA_WORKLOADS, WORKLOADS, LosaWorkload, Workload, get_workload  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_base,
    make_losa_base,
    make_losa_cache,
    make_losa_iteration,
    make_step,
    score_jump,
    tiny_random,
)
