"""MI355X-native hot path of the Fast-weight Product Key Memory (FwPKM) layer.

The layer's work runs in hand-written HIP kernels for gfx950 behind a C-ABI
library (``libfwpkm.so``, declared in ``include/fwpkm.h``).  This package
holds the kernel sources (``csrc/``), the build step (``build.py``), a thin
ctypes binding with the library's entry-point names (``fwpkm.py``), and the
seeded synthetic workloads (``workloads.py``).
"""
from .workloads import FwpkmConfig, WORKLOADS, make_state, make_tokens, make_workload  # noqa: F401
