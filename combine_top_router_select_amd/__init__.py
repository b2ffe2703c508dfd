"""Per-GPU MoE expert-parallel dispatch and combine for AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libmoe_route.so``, declared in ``include/moe_route.h``).  ``ops`` is a thin
ctypes binding with the same entry-point names; ``workloads`` draws the seeded
synthetic inputs.  Importing the package loads nothing: the library is opened
on first use and its absence raises an error.
"""
__all__ = ["ops", "workloads"]
