"""Seeded synthetic workloads for the per-rank shard step.

This package is shared by the oracle tests, the GPU parity tests and the
benchmark.  It holds only workload descriptions (shapes, world sizes,
hyperparameters) and seeded random-number draws; none of the method's
arithmetic (packing, reduction, optimizer update, rounding) lives here.
"""

from .configs import CONFIGS, Config, transformer_unit_shapes, c5_tensor_sizes  # noqa: F401
from . import gen  # noqa: F401
