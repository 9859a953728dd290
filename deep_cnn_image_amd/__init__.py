"""AlexNet forward pass and training step on MI355X (gfx950).

The compute lives in libalexnet.so (HIP kernels behind a C ABI, declared in
include/alexnet.h); ``binding`` mirrors that ABI one function per entry point,
``session`` holds torch-allocated device buffers, ``inputs`` draws the seeded
synthetic workloads.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
