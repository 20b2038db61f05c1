"""MI355X-native W4A4G4 triple-branch quantized linear (FourTune).

The compute path lives in libft.so (hand-written HIP kernels for gfx950,
C ABI in include/ft.h).  This package only marshals torch tensors into that
ABI (``ops``) and wraps the layer for autograd (``linear``).
"""
from . import _lib  # noqa: F401

__all__ = ["ops", "build"]
