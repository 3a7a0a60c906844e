"""Seeded synthetic inputs for the IndexMem / MomentKV hot path.

This package is shared by the fp64 oracle's tests and by the GPU path's tests and
benchmark.  It holds workload shapes, seeded random draws and number-format
conversions (bf16 <-> float) only; none of the method's arithmetic lives here.
"""
from .configs import WORKLOADS, Config, workload  # noqa: F401
from . import gen  # noqa: F401
