"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds input construction only (random draws, the low-rank key structure,
forced ties made by duplicating keys) and none of the attention arithmetic.
"""
from .inputs import WORKLOADS, Workload, generate, workload  # noqa: F401
