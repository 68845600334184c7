"""Seeded synthetic inputs shared by the oracle's tests and the HIP path."""
from .workload import *  # noqa: F401,F403
