"""Shared-prefix decode attention over a paged radix-tree KV cache, for
AMD MI355X (gfx950).  The compute path is the C-ABI library ``libcap.so``
(hand-written HIP kernels); ``cap`` is its thin ctypes binding and
``workloads`` builds seeded synthetic inputs.  Importing the package loads
nothing; the library is loaded on first use and its absence is an error.
"""
