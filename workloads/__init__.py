"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle checks."""
from .configs import WORKLOADS, Workload  # noqa: F401
from .gen import make_inputs, torch_dtype  # noqa: F401
