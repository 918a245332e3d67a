"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .workloads import *  # noqa: F401,F403
