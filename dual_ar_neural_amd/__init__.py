"""dual_ar_neural_amd: the Fast-AR codebook decoder of the Dual-AR TTS model
as a gfx950 (MI355X) HIP library.

The compute lives in libs2fast.so (C ABI: include/s2fast.h); this package
only builds it (``build``) and marshals torch tensors into it (``binding``).
"""
from .binding import FastAR, S2FastError, library, device_weights, rope_table, sample  # noqa: F401
