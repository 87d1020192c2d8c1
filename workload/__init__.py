"""Seeded synthetic SFI decode workloads (sizes, knobs and input generators only)."""
from .configs import WORKLOADS, ORDER, BENCH_WORKLOAD, Workload, get  # noqa: F401
