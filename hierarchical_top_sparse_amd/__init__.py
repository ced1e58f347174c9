"""MI355X-native Log-linear Sparse Attention (LLSA).

The hot path runs in libllsa.so (hand-written HIP kernels for gfx950 behind a C ABI, declared
in include/llsa.h).  `_abi` binds every C entry point under the same name; `ops` chains them
into the forward/backward op.  Nothing here loads the library until a call needs it.
"""
__all__ = ["ops", "_abi", "gen"]
