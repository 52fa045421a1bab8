"""H-BitLinear (BitNet v2) forward on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libhbl.so`` built from ``csrc/`` (hand-written HIP
kernels); ``binding`` marshals torch tensors into it.  Importing this package does not load
the library; ``binding.lib()`` does, and raises if it is missing.
"""
__all__ = ["binding", "inputs"]
