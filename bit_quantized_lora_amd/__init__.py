"""MI355X-native W4A4G4 triple-branch quantized linear (FourTune).

The compute path lives in libft.so (hand-written HIP kernels for gfx950,
C ABI in include/ft.h).  ``ops`` marshals torch tensors into that ABI and
``linear.Linear`` wraps the forward and backward entry points as a torch
module whose only trainable parameters are the LoRA factors.
"""
from . import _lib  # noqa: F401

__all__ = ["ops", "linear", "build"]
