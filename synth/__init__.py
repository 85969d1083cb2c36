"""Seeded synthetic decode workloads (shapes, parameters and inputs).

Shared by the tests, the benchmark and the oracle checks; holds none of the
decode method's arithmetic.
"""
from . import configs, gen  # noqa: F401
