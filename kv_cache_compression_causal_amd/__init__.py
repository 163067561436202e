"""LightTransfer-Test hot path on MI355X (gfx950): HIP kernels behind a C ABI.

* ``api``   -- thin ctypes binding of include/lt.h (same names as the C calls);
* ``ops``   -- allocating conveniences on top of ``api``;
* ``synth`` -- seeded synthetic inputs shaped like the pages' workloads;
* ``build`` -- compiles liblt.so with hipcc for gfx950.

Importing the package loads nothing; the library is loaded on first use and
its absence is an error (there is no fallback path).
"""
__all__ = ["api", "ops", "synth", "build"]
