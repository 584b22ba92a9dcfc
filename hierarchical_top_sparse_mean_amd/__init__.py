"""MI355X (gfx950) Log-linear Sparse Attention: HIP kernels behind a C ABI.

``llsa`` is the ctypes binding of ``libllsa.so``; ``inputs`` draws the seeded
synthetic workloads; ``build`` compiles the library.
"""
