"""MI355X (gfx950) Compass/Cohere2 parallel decoder layer.

The compute lives in libcompass.so (hand-written HIP kernels behind the C ABI in
include/compass.h); `binding` is its ctypes wrapper. Importing the package does
not load the library; importing `cohere2_block_mrope_amd.binding` does, and
fails loudly if it has not been built.
"""
__all__ = ["binding"]
