"""Seeded synthetic workloads for large-beam GDN decoding.

Shared by the GPU path's harness and the CPU oracle; holds sizes, seeds and
random draws only.
"""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from . import gen  # noqa: F401
