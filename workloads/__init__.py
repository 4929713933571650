"""Seeded synthetic workloads shared by the oracle tests and the HIP path.

Holds shapes, distributions and random draws only -- no step of the method.
"""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from . import synth  # noqa: F401
