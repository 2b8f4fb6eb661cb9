"""LiftQuant lift-then-project linear layer on MI355X (gfx950).

The compute path is the HIP library ``liblq.so`` behind the C ABI declared in
``include/lq.h``; ``bit_lifted_gemv_amd.lq`` is a thin ctypes binding to it.
Importing this package loads nothing; the library is opened on first use.
"""
__all__ = ["synth"]
