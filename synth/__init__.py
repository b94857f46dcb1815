"""Seeded synthetic inputs for the Graft per-step path.

This package is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It draws random numbers and lays out inputs; it computes none
of the method's own arithmetic (no pruning, retrieval, flattening, top-k,
acceptance or matrix update).
"""
from .configs import WORKLOADS, GraftConfig, get  # noqa: F401
