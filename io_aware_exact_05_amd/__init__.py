"""Exact attention forward pass for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(``include/fa.h``, ``libfa.so``).  ``io_aware_exact_05_amd.fa`` is the thin
ctypes binding with the same entry-point names; ``inputs`` draws the seeded
synthetic workloads.
"""
__all__ = ["fa", "inputs"]
