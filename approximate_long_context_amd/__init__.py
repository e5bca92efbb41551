"""Positional-LSH approximation of ALiBi attention for AMD MI355X (gfx950).

The estimator and its kernels live in libplsh.so (C ABI: include/plsh.h);
`plsh` is the thin ctypes binding (the library is loaded on first use);
`workloads` holds the seeded input recipes.
"""

from . import plsh, workloads  # noqa: F401

__all__ = ["plsh", "workloads"]
