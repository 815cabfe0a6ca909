"""Seeded synthetic inputs shared by the oracle side and the HIP side (inputs only)."""
from .inputs import *  # noqa: F401,F403
from .inputs import WORKLOADS, Workload  # noqa: F401
