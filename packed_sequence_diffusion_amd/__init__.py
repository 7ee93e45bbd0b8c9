"""Packed-sequence diffusion-transformer block for AMD Instinct MI355X.

The compute lives in ``libdit.so`` (hand-written HIP kernels for gfx950 behind
the C ABI in include/dit.h); ``packed_sequence_diffusion_amd.dit`` is its
ctypes binding.  Build with ``python -m packed_sequence_diffusion_amd.build``.
"""

__all__ = ["dit"]
