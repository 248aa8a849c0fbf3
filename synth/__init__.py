"""Seeded synthetic inputs shared by the CPU oracle and the HIP path (no attention arithmetic)."""
from .gen import *  # noqa: F401,F403
from .gen import Workload, make_config, make_custom  # noqa: F401
