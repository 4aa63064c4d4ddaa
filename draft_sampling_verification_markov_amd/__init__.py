"""MI355X (gfx950) implementation of the per-cycle draft -> schedule -> verify
step of confidence-scheduled speculative decoding with a Markov draft head.

The work is done by ``libdspark.so`` (HIP kernels behind a C ABI declared in
include/dspark.h); ``dspark`` is its ctypes binding and ``runner`` allocates
the caller-owned buffers with torch.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
__all__ = ["dspark", "runner", "build"]
