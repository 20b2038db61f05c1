"""ctypes loader for libft.so (the C ABI declared in include/ft.h).

The library must be built (``__graft_entry__.build()`` or
``python -m bit_quantized_lora_amd.build``); loading fails loudly otherwise.
There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int32, c_int64, c_size_t, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libft.so")

FT_OK, FT_EINVAL, FT_ESHAPE, FT_EALIGN, FT_EHIP, FT_ENOTSUP, FT_ESPACE = range(7)
FT_SCALE_POW2, FT_SCALE_F32 = 0, 1
FT_OUT_F32, FT_OUT_BF16 = 0, 1
FT_NOALLOC_SCRATCH_BYTES = 32 << 20

# name -> argtypes (restype is ft_status = int unless stated)
_SIGS = {
    "ft_quant_block16": [c_void_p, c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
    "ft_quant_block16_op": [c_void_p, c_int64, c_int64, c_int64] + [c_void_p] * 9,
    "ft_operand_bytes": [c_int64, c_int64],
    "ft_operand_scale_bytes": [c_int64, c_int64],
    "ft_lowrank_fused": [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                         c_void_p, c_size_t, c_void_p],
    "ft_lowrank_workspace": [c_int64, c_int64, c_int32],
    "ft_lowrank_plan": [c_int64, c_int64, c_int32, c_void_p],
    "ft_quant_lowrank": [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_quant_lowrank_db": [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_quant_lowrank_db_workspace": [c_int64, c_int64, c_int32, c_int32],
    "ft_gelu_quant_lowrank": [c_void_p, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_linear_fwd": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                      c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "ft_linear_fwd_ws": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                         c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_size_t,
                         c_void_p],
    "ft_linear_fwd_workspace": [c_int64, c_int64, c_int64],
    "ft_linear_plan": [c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p],
    "ft_linear_fwd_gelu": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                           c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                           c_void_p],
    "ft_linear_bwd": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                      c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                      c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_linear_bwd_workspace": [c_int64, c_int64, c_int64, c_int32],
    "ft_linear_bwd_plan": [c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p],
    "ft_linear_bwd_noalloc": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_int32, c_void_p, c_void_p, c_void_p],
    "ft_linear_fwd_op": [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                         c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "ft_linear_bwd_op": [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                         c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                         c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_linear_fwd_a16": [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                          c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "ft_linear_bwd_g16": [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                          c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                          c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_quant_group": [c_void_p, c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p],
    "ft_requant_group_t": [c_void_p, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p],
    "ft_linear_fwd_grp": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                          c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "ft_linear_bwd_grp": [c_int64, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                          c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                          c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "ft_gelu_fwd": [c_void_p, c_int64, c_void_p, c_void_p],
    "ft_gelu_bwd": [c_void_p, c_void_p, c_int64, c_void_p, c_void_p],
    "ft_stream_2to1": [c_void_p, c_int64, c_void_p, c_void_p],
    "ft_status_str": [c_int32],
}
_RESTYPES = {"ft_operand_bytes": c_size_t, "ft_quant_lowrank_db_workspace": c_size_t, "ft_operand_scale_bytes": c_size_t,
             "ft_linear_bwd_workspace": c_size_t, "ft_linear_fwd_workspace": c_size_t,
             "ft_lowrank_workspace": c_size_t, "ft_status_str": c_char_p}

_lib = None


class FtError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().ft_status_str(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libft.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() "
                "(hipcc --offload-arch=gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name, None)
            if f is None:
                continue
            f.argtypes = args
            f.restype = _RESTYPES.get(name, c_int32)
        _lib = L
    return _lib


def exported_symbols():
    """Names from the ABI table that the loaded library exports."""
    L = lib()
    return [n for n in _SIGS if getattr(L, n, None) is not None]


def check(fn: str, status: int) -> None:
    if status != FT_OK:
        raise FtError(fn, status)
