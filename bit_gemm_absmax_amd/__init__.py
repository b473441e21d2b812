"""BitLinear W1.58A8 on MI355X (gfx950): a C-ABI HIP library and its binding.

Import of this package does not load the HIP library; the binding in
:mod:`bit_gemm_absmax_amd.bitlinear` loads it on first use and raises if it is
missing.
"""
__all__ = ["synth"]
