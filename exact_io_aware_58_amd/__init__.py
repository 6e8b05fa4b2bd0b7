"""FlashAttention fused exact attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libfa.so`` (hand-written HIP kernels
in ``csrc/``), reached through the thin ctypes binding in ``fa.py``.  Importing
the package loads nothing; ``exact_io_aware_58_amd.fa`` loads the library and
raises if it has not been built.
"""
__all__ = ["fa", "inputs"]
