"""Seeded synthetic MoE routing workloads.

This package only draws inputs (hidden rows, top-k expert ids, top-k weights).
It holds none of the dispatch/combine arithmetic, so both the CPU oracle and
the HIP path can consume the same arrays without sharing any method code.
"""

from .workloads import (  # noqa: F401
    balanced_routing,
    CONFIGS,
    Workload,
    WorkloadSpec,
    make_workload,
    make_routing,
    make_hidden,
    spec,
)
