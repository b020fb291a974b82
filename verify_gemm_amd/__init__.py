"""verify_gemm_amd: the NVFP4 decode / speculative-verify weight pass on
MI355X (gfx950).

The product is ``libvgemm.so`` (C ABI in ``include/vgemm.h``), built from the
HIP sources in ``csrc/``; ``binding`` is its thin ctypes wrapper for torch
device tensors, and ``synth`` draws the seeded synthetic workloads.  Importing
this package loads nothing; the binding loads the library on first use and
raises if it is not built.
"""
__all__ = ["binding", "synth", "build"]
