"""Seeded synthetic inputs shared by the oracle-side and GPU-side tests and
the bench. Holds no attention arithmetic."""

from .gen import BF16, F32, BUILDERS, Workload, WriteOp, build, make_values, tail_waste  # noqa: F401
from .pool import HostBlockPool, PoolExhausted  # noqa: F401
