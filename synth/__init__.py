"""Seeded synthetic inputs (generator + workload shapes), shared by the oracle side and
the GPU side; contains none of the decode method's arithmetic."""
from . import gen, workloads  # noqa: F401
