"""SANTA stochastic sparse decode-step attention for MI355X (gfx950).

The compute path is the C-ABI library ``libsanta.so`` built from ``csrc/``
(hand-written HIP kernels).  ``santa`` is a thin ctypes binding with the same
entry-point names; it only marshals pointers, sizes and the HIP stream.
``workloads`` draws seeded synthetic inputs.

Importing this package does not load the library; ``santa`` loads it on first
use and raises if it has not been built.
"""

__all__ = ["santa", "workloads", "build"]
