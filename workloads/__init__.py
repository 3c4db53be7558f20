"""Seeded synthetic workloads (inputs only; none of the method's arithmetic)."""
from .gen import *  # noqa: F401,F403
from .gen import WORKLOADS, Workload  # noqa: F401
