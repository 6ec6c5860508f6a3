"""Paged decode attention and the KV-cache scatter for MI355X (gfx950).

The compute path is the C-ABI library ``libpa.so`` built from ``csrc/``
(hand-written HIP kernels); ``lib`` is its thin ctypes binding and
``workloads`` builds seeded synthetic batches. The library is loaded on
first use; a missing or unbuilt library raises instead of falling back.
"""

__all__ = ["lib", "workloads"]
