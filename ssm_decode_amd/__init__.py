"""SketchSSM decode hot path on MI355X (gfx950).

``abi``      ctypes binding of libsketchssm.so (the C ABI in include/sketchssm.h)
``layer``    torch-allocated device buffers of one layer and the ABI structs
``feed``     moves seeded synthetic inputs into device buffers
``traffic``  algorithmic byte model of the decode path
``build``    compiles the HIP library in-tree
"""
from . import abi  # noqa: F401

__all__ = ["abi"]
