"""Block-sparse spatiotemporal attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libfva.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/fva.h``); ``fva`` is its thin ctypes binding and
``synth`` the seeded input generator.  Importing the package loads nothing;
the library is opened on first use of ``fva``.
"""
