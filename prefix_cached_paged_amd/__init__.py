"""librax: paged-KV EXTEND / DECODE attention for AMD MI355X (gfx950).

The compute lives in the C-ABI shared library ``librax.so`` (hand-written HIP
kernels); ``prefix_cached_paged_amd.rax`` is a thin ctypes binding over it.
``workloads`` draws the seeded synthetic inputs and ``accounting`` counts the
algorithmic work used in the roofline figures.

Importing this package loads nothing; the binding loads the library on first use
and raises if it has not been built.
"""

__all__ = ["rax", "workloads", "accounting", "device"]
