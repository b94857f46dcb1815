"""Graft per-step hot path on AMD Instinct MI355X (gfx950).

libgraft.so (HIP kernels + C ABI, include/graft.h) does all the work; this
package is its Python binding (``_lib``), the build script (``build``) and a
device-resident step driver (``driver.GraftPipeline``).
"""
from ._lib import load  # noqa: F401

__all__ = ["load"]
