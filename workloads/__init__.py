"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This package holds workload shapes and random draws only: no step of the
method (no page map, no filter, no reshard, no attention, no merge).  Both the
float64 oracle and the HIP path consume what it produces; neither is imported
here.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from . import gen  # noqa: F401
