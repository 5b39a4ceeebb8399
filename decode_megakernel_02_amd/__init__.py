"""MI355X (gfx950) single-launch decode for Llama-style decoders.

The whole greedy decode step runs as one persistent HIP kernel (libmk.so,
C ABI in include/mk.h); `mk` is its ctypes binding.
"""
from . import mk  # noqa: F401
