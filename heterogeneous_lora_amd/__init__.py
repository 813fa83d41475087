"""Heterogeneous batched LoRA on MI355X (gfx950): paged adapter pool, MBGMV decode
kernels and SGMV (MFMA) prefill kernels behind the C ABI in include/slora.h.

`_lib` is the ctypes binding of libslora.so; `runtime` is the torch plumbing
(device memory, pinned host memory, streams) used by tests and benchmarks.
Importing the package does not load the library; `_lib.load()` does, and fails
loudly if the library has not been built.
"""

__all__ = ["_lib", "runtime", "build"]
