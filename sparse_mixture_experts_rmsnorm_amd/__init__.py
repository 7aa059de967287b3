"""MI355X-native forward pass of one sparse MoE FFN layer.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libmoe_mi355x.so``, declared in ``include/moe.h``); this package is
its thin ctypes binding plus the workload shapes and the seeded synthetic
input generator.  Importing the package does not load the library; the first
call into it does, and raises if the library has not been built.
"""
from .workloads import WORKLOADS, Workload  # noqa: F401
