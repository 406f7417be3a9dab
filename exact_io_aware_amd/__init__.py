"""Exact IO-aware tiled attention for the AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``include/fa.h``); ``exact_io_aware_amd.fa`` is a thin ctypes binding over it
that marshals torch tensors into device pointers and the current HIP stream.
The library is loaded on first use; if it has not been built, every entry
point raises instead of falling back to any other implementation.
"""

__all__ = ["fa", "workloads"]
