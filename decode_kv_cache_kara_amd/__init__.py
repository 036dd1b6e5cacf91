"""Kara decode-time KV-cache compression on AMD Instinct MI355X (gfx950).

The compression step runs in libkara.so (HIP kernels behind the C ABI of
include/kara.h); ``kara`` is its ctypes binding, ``synth`` draws seeded
synthetic workloads, ``runner`` holds device buffers for repeated calls.
Importing ``kara`` fails if the library has not been built.
"""

__all__ = ["kara", "synth", "runner"]
