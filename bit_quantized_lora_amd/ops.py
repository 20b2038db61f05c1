"""Thin torch binding of the ft C ABI (argument marshalling only).

Each function takes CUDA (HIP) tensors, allocates outputs with torch (device
memory is torch's job here), passes raw pointers and the current stream to
libft.so and raises ``FtError`` on a non-OK status.  No arithmetic of the
method happens in Python.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import check, lib

_MODES = {"pow2": _lib.FT_SCALE_POW2, "f32": _lib.FT_SCALE_F32}
_OUT = {torch.float32: _lib.FT_OUT_F32, torch.bfloat16: _lib.FT_OUT_BF16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, dtype, name: str, shape=None, contiguous: bool = True, min_numel: int = 0, used: bool = True) -> None:
    """Check a tensor before its pointer crosses the ABI: dtype, shape,
    contiguity and size (the device is checked by _same_device once every
    tensor of a call has passed these).  Raises ValueError on a mismatch."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if not used and t.numel() == 0:
        return   # an operand the call does not read (its product is empty) may be empty
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(s) for s in shape):
        # an empty operand (a zero-sized dimension) may come in any empty shape
        if not (t.numel() == 0 and math.prod(int(s) for s in shape) == 0):
            raise ValueError(f"{name} must have shape {tuple(int(s) for s in shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")


def _need_matrix(x, name: str, rows=None, cols=None) -> None:
    """A bf16 input matrix read with a leading dimension: 2-D, unit column stride,
    rows 16-byte aligned."""
    _need(x, torch.bfloat16, name, contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1 or (x.shape[0] > 1 and x.stride(0) < x.shape[1]):
        raise ValueError(f"{name} must be a 2-D matrix with unit column stride")
    if rows is not None and (x.shape[0] != rows or x.shape[1] != cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(x.shape)}")


def _mult16(name: str, *dims) -> None:
    for d in dims:
        if d < 0 or d % 16:
            raise ValueError(f"{name}: dimensions must be non-negative multiples of 16, got {dims}")


def _same_device(*ts) -> None:
    """Every tensor of a call on the same GPU device."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor must be a device tensor")
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _ws(workspace, nbytes: int, dev, name: str = "workspace"):
    """Caller workspace checked against the required size, or a fresh one."""
    if workspace is None:
        return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, name, min_numel=nbytes)
    return workspace


class Prepared:
    """A library call whose tensors were checked once.  Calling the object issues
    the same call on the same buffers, on the device's current stream, with no
    further Python-side checks (for loops that run one step many times).  The
    tensors it was prepared with are kept alive by the object and must keep their
    shapes; their contents may change between calls."""

    __slots__ = ("_fn", "_name", "_args", "_dev", "result", "_keep")

    def __init__(self, name: str, args: tuple, dev, result, keep):
        self._fn = getattr(lib(), name)
        self._name, self._args, self._dev, self.result, self._keep = name, args, dev, result, keep

    def __call__(self):
        st = self._fn(*self._args, torch.cuda.current_stream(self._dev).cuda_stream)
        if st != _lib.FT_OK:
            raise _lib.FtError(self._name, st)
        return self.result


def _issue(name: str, args: tuple, dev, result, keep, prepare: bool):
    if prepare:
        return Prepared(name, args, dev, result, keep)
    st = getattr(lib(), name)(*args, torch.cuda.current_stream(dev).cuda_stream)
    check(name, st)
    return result


def quant_block16(x: torch.Tensor, mode: str = "pow2", rm: bool = True, cm: bool = False,
                  out: Optional[Tuple] = None, scales_cm: bool = False):
    """Q(x) for a bf16 [rows, cols] matrix -> (codes_rm, codes_cm, scales), plus
    the transposed scale grid as a fourth element when ``scales_cm`` is set.

    ``out`` may supply preallocated (codes_rm, codes_cm, scales[, scales_cm]) buffers.
    """
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    _need_matrix(x, "x")
    rows, cols = x.shape
    _mult16("quant_block16", rows, cols)
    dev = x.device
    sdt = torch.uint8 if mode == "pow2" else torch.float32
    if out is not None:
        codes_rm, codes_cm, scales = out[:3]
        sc_cm = out[3] if len(out) > 3 else None
    else:
        codes_rm = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev) if rm else None
        codes_cm = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev) if cm else None
        scales = torch.empty((rows // 16, cols // 16), dtype=sdt, device=dev)
        sc_cm = torch.empty((cols // 16, rows // 16), dtype=sdt, device=dev) if scales_cm else None
    if codes_rm is None and codes_cm is None:
        raise ValueError("at least one code layout is required")
    if codes_rm is not None:
        _need(codes_rm, torch.uint8, "codes_rm", (rows, cols // 2))
    if codes_cm is not None:
        _need(codes_cm, torch.uint8, "codes_cm", (cols, rows // 2))
    _need(scales, sdt, "scales", (rows // 16, cols // 16))
    if sc_cm is not None:
        _need(sc_cm, sdt, "scales_cm", (cols // 16, rows // 16))
    _same_device(x, codes_rm, codes_cm, scales, sc_cm)
    st = lib().ft_quant_block16(x.data_ptr(), rows, cols, x.stride(0), _MODES[mode],
                                _ptr(codes_rm), _ptr(codes_cm), scales.data_ptr(), _ptr(sc_cm),
                                _stream(x))
    check("ft_quant_block16", st)
    if sc_cm is not None:
        return codes_rm, codes_cm, scales, sc_cm
    return codes_rm, codes_cm, scales


def operand_shapes(rows: int, cols: int):
    """((rows, bytes per row), (rows/16, scale bytes per row)) of the operand of a [rows, cols] matrix."""
    n = int(lib().ft_operand_bytes(rows, cols))
    ns = int(lib().ft_operand_scale_bytes(rows, cols))
    return (rows, n // rows if rows else 0), (rows // 16, ns // (rows // 16) if rows >= 16 else 0)


def quant_block16_op(x: torch.Tensor, codes_rm: bool = False, codes_cm: bool = False, op_rm: bool = True,
                     op_cm: bool = False, out: Optional[dict] = None) -> dict:
    """Q(x) (power-of-two scales) -> dict with any of "codes_rm", "codes_cm", "scales",
    "op_rm", "op_rm_scales" (the operand of x), "op_cm", "op_cm_scales" (of x^T).

    ``out`` may supply preallocated buffers under the same keys."""
    _need_matrix(x, "x")
    rows, cols = x.shape
    _mult16("quant_block16_op", rows, cols)
    dev = x.device
    u8 = torch.uint8
    if out is None:
        out = {}
        if codes_rm:
            out["codes_rm"] = torch.empty((rows, cols // 2), dtype=u8, device=dev)
        if codes_cm:
            out["codes_cm"] = torch.empty((cols, rows // 2), dtype=u8, device=dev)
        if codes_rm or codes_cm:
            out["scales"] = torch.empty((rows // 16, cols // 16), dtype=u8, device=dev)
        if op_rm:
            (a, b), (c, d) = operand_shapes(rows, cols)
            out["op_rm"] = torch.empty((a, b), dtype=u8, device=dev)
            out["op_rm_scales"] = torch.empty((c, d), dtype=u8, device=dev)
        if op_cm:
            (a, b), (c, d) = operand_shapes(cols, rows)
            out["op_cm"] = torch.empty((a, b), dtype=u8, device=dev)
            out["op_cm_scales"] = torch.empty((c, d), dtype=u8, device=dev)
    shapes = {"codes_rm": (rows, cols // 2), "codes_cm": (cols, rows // 2), "scales": (rows // 16, cols // 16),
              "scales_cm": (cols // 16, rows // 16)}
    if "op_rm" in out or "op_rm_scales" in out:
        shapes["op_rm"], shapes["op_rm_scales"] = operand_shapes(rows, cols)
    if "op_cm" in out or "op_cm_scales" in out:
        shapes["op_cm"], shapes["op_cm_scales"] = operand_shapes(cols, rows)
    for k, t in out.items():
        if k not in shapes:
            raise ValueError(f"unknown output {k!r}")
        _need(t, u8, k, shapes[k])
    _same_device(x, *out.values())
    g = lambda k: _ptr(out.get(k))
    st = lib().ft_quant_block16_op(x.data_ptr(), rows, cols, x.stride(0), g("codes_rm"), g("codes_cm"),
                                   g("scales"), g("scales_cm"), g("op_rm"), g("op_rm_scales"), g("op_cm"),
                                   g("op_cm_scales"), _stream(x))
    check("ft_quant_block16_op", st)
    return out


def lowrank_workspace(M: int, Kin: int, rho: int) -> int:
    return int(lib().ft_lowrank_workspace(M, Kin, rho))


def _factors(wa, wb, Kin: int, names=("wa", "wb")):
    """Rank-major bf16 factors [rank, Kin]: returns (ra, rb)."""
    for w, n in ((wa, names[0]), (wb, names[1])):
        _need(w, torch.bfloat16, n)
        if w.dim() != 2 or w.shape[1] != Kin:
            raise ValueError(f"{n} must be contiguous [rank, {Kin}], got {tuple(w.shape)}")
    ra, rb = wa.shape[0], wb.shape[0]
    _mult16("ranks", ra, rb)
    if ra + rb > 128:
        raise ValueError(f"ranks {ra} + {rb} exceed 128")
    return ra, rb


def lowrank_fused(inp: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = [inp wa^T | inp wb^T] in fp32; wa [ra, Kin], wb [rb, Kin] bf16."""
    _need_matrix(inp, "inp")
    M, Kin = inp.shape
    _mult16("lowrank_fused", M, Kin)
    ra, rb = _factors(wa, wb, Kin)
    if out is None:
        out = torch.empty((M, ra + rb), dtype=torch.float32, device=inp.device)
    _need(out, torch.float32, "out", (M, ra + rb))
    workspace = _ws(workspace, lowrank_workspace(M, Kin, ra + rb), inp.device)
    _same_device(inp, wa, wb, out, workspace)
    st = lib().ft_lowrank_fused(inp.data_ptr(), M, Kin, inp.stride(0), wa.data_ptr(), ra,
                                wb.data_ptr(), rb, out.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream(inp))
    check("ft_lowrank_fused", st)
    return out


def quant_lowrank(inp: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor, out: Optional[torch.Tensor] = None,
                  codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """(out, codes_rm, scales): [inp wa^T | inp wb^T] and Q(inp) in one read of inp.
    With ``prepare`` the checked call is returned as a ``Prepared`` object instead."""
    _need_matrix(inp, "inp")
    M, Kin = inp.shape
    _mult16("quant_lowrank", M, Kin)
    ra, rb = _factors(wa, wb, Kin)
    dev = inp.device
    if out is None:
        out = torch.empty((M, ra + rb), dtype=torch.float32, device=dev)
    if codes is None:
        codes = torch.empty((M, Kin // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M // 16, Kin // 16), dtype=torch.uint8, device=dev)
    _need(out, torch.float32, "out", (M, ra + rb))
    _need(codes, torch.uint8, "codes", (M, Kin // 2))
    _need(scales, torch.uint8, "scales", (M // 16, Kin // 16))
    workspace = _ws(workspace, lowrank_workspace(M, Kin, ra + rb), dev)
    _same_device(inp, wa, wb, out, codes, scales, workspace)
    args = (inp.data_ptr(), M, Kin, inp.stride(0), wa.data_ptr(), ra, wb.data_ptr(), rb, out.data_ptr(),
            codes.data_ptr(), scales.data_ptr(), workspace.data_ptr(), workspace.numel())
    return _issue("ft_quant_lowrank", args, inp.device, (out, codes, scales),
                  (inp, wa, wb, out, codes, scales, workspace), prepare)


def quant_lowrank_db_workspace(M: int, Kin: int, rho: int, r: int) -> int:
    return int(lib().ft_quant_lowrank_db_workspace(M, Kin, rho, r))


def quant_lowrank_db(g: torch.Tensor, L2: torch.Tensor, B: torch.Tensor, T: torch.Tensor,
                     out: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """(V, codes_rm, scales, dB): the backward's pass over G with dB = T[:, rs:]^T G
    folded in (T: the forward's [M, rs + r]).  ``prepare``: return a ``Prepared`` call."""
    _need_matrix(g, "g")
    M, N = g.shape
    _mult16("quant_lowrank_db", M, N)
    rs, r = _factors(L2, B, N, names=("L2", "B"))
    dev = g.device
    if out is None:
        out = torch.empty((M, rs + r), dtype=torch.float32, device=dev)
    if codes is None:
        codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M // 16, N // 16), dtype=torch.uint8, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    _need(out, torch.float32, "out", (M, rs + r))
    _need(codes, torch.uint8, "codes", (M, N // 2))
    _need(scales, torch.uint8, "scales", (M // 16, N // 16))
    _need(T, torch.float32, "T", (M, rs + r))
    _need(dB, torch.float32, "dB", (r, N))
    workspace = _ws(workspace, quant_lowrank_db_workspace(M, N, rs + r, r), dev)
    _same_device(g, L2, B, T, out, codes, scales, dB, workspace)
    args = (g.data_ptr(), M, N, g.stride(0), L2.data_ptr(), rs, B.data_ptr(), r, out.data_ptr(), codes.data_ptr(),
            scales.data_ptr(), T.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel())
    return _issue("ft_quant_lowrank_db", args, dev, (out, codes, scales, dB),
                  (g, L2, B, T, out, codes, scales, dB, workspace), prepare)


def gelu_quant_lowrank(y: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor, out=None, workspace=None):
    """h = GELU(y), Q(h) and [h wa^T | h wb^T] from one read of y:
    returns (h, T, codes, scales)."""
    _need(y, torch.bfloat16, "y")
    if y.dim() != 2:
        raise ValueError("y must be a 2-D matrix")
    M, Kin = y.shape
    _mult16("gelu_quant_lowrank", M, Kin)
    ra, rb = _factors(wa, wb, Kin)
    dev = y.device
    if out is None:
        out = (torch.empty((M, Kin), dtype=torch.bfloat16, device=dev),
               torch.empty((M, ra + rb), dtype=torch.float32, device=dev),
               torch.empty((M, Kin // 2), dtype=torch.uint8, device=dev),
               torch.empty((M // 16, Kin // 16), dtype=torch.uint8, device=dev))
    h, T, codes, scales = out
    _need(h, torch.bfloat16, "h", (M, Kin))
    _need(T, torch.float32, "T", (M, ra + rb))
    _need(codes, torch.uint8, "codes", (M, Kin // 2))
    _need(scales, torch.uint8, "scales", (M // 16, Kin // 16))
    workspace = _ws(workspace, lowrank_workspace(M, Kin, ra + rb), dev)
    _same_device(y, wa, wb, h, T, codes, scales, workspace)
    st = lib().ft_gelu_quant_lowrank(y.data_ptr(), M, Kin, wa.data_ptr(), ra, wb.data_ptr(), rb, h.data_ptr(),
                                     T.data_ptr(), codes.data_ptr(), scales.data_ptr(), workspace.data_ptr(),
                                     workspace.numel(), _stream(y))
    check("ft_gelu_quant_lowrank", st)
    return h, T, codes, scales


def _out_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _OUT:
        raise ValueError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    return _OUT[t.dtype]


def _up_factors(L2, B, N: int, names=("L2", "B")):
    """Rank-major bf16 up-projection factors [rank, N]: returns (rs, r)."""
    for w, n in ((L2, names[0]), (B, names[1])):
        _need(w, torch.bfloat16, n)
        if w.dim() != 2 or w.shape[1] != N:
            raise ValueError(f"{n} must be contiguous [rank, {N}], got {tuple(w.shape)}")
    rs, r = L2.shape[0], B.shape[0]
    _mult16("ranks", rs, r)
    if rs + r > 128:
        raise ValueError(f"ranks {rs} + {r} exceed 128")
    return rs, r


def _sdt(mode: str):
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    return torch.uint8 if mode == "pow2" else torch.float32


def linear_fwd_workspace(M: int, N: int, K: int) -> int:
    return int(lib().ft_linear_fwd_workspace(M, N, K))


def linear_plan(M: int, N: int, K: int, backward: bool = False, with_ws: bool = True):
    """(tile rows, tile columns, reduction splits) of the 4-bit GEMM of
    linear_fwd (backward False) or of linear_bwd's dX GEMM (backward True)."""
    import ctypes
    out = (ctypes.c_int32 * 3)()
    check("ft_linear_plan", lib().ft_linear_plan(M, N, K, int(backward), int(with_ws), ctypes.addressof(out)))
    return int(out[0]), int(out[1]), int(out[2])


def linear_fwd(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
               out_dtype=torch.float32, mode: str = "pow2", out: Optional[torch.Tensor] = None,
               prepare: bool = False, split: bool = True, workspace: Optional[torch.Tensor] = None):
    """Y = deq(Xq) deq(Rq)^T + T[:, :rs] L2 + T[:, rs:] B (``prepare``: return a ``Prepared`` call).

    ``split``: shapes with too few output tiles for the GPU split their reduction
    (ft_linear_fwd_ws, with ``workspace`` or a fresh one); False: ft_linear_fwd,
    never split."""
    _mult16("linear_fwd", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    sdt = _sdt(mode)
    rs, r = _up_factors(L2, B, N)
    _need(xq_codes, torch.uint8, "xq_codes", (M, K // 2), used=gemm)
    _need(xq_scales, sdt, "xq_scales", (M // 16, K // 16), used=gemm)
    _need(rq_codes, torch.uint8, "rq_codes", (N, K // 2), used=gemm)
    _need(rq_scales, sdt, "rq_scales", (N // 16, K // 16), used=gemm)
    _need(T, torch.float32, "T", (M, rs + r))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    odt = _out_dtype(out, "out")
    _need(out, out.dtype, "out", (M, N))
    need = linear_fwd_workspace(M, N, K) if split else 0
    if need:
        workspace = _ws(workspace, need, T.device)
    _same_device(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, out, workspace if need else None)
    args = (M, N, K, _MODES[mode], xq_codes.data_ptr(), xq_scales.data_ptr(), rq_codes.data_ptr(),
            rq_scales.data_ptr(), T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r, out.data_ptr(), odt)
    keep = (xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, out)
    if need:
        return _issue("ft_linear_fwd_ws", args + (workspace.data_ptr(), workspace.numel()), T.device, out,
                      keep + (workspace,), prepare)
    return _issue("ft_linear_fwd", args, T.device, out, keep, prepare)


def linear_fwd_gelu(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
                    mode: str = "pow2", out=None):
    """First linear of an MLP with the fused epilogue: Y (bf16), H = GELU(Y) (bf16)
    and Q(H) (row-major codes, scales); returns (Y, H, h_codes, h_scales)."""
    _mult16("linear_fwd_gelu", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    sdt = _sdt(mode)
    rs, r = _up_factors(L2, B, N)
    _need(xq_codes, torch.uint8, "xq_codes", (M, K // 2), used=gemm)
    _need(xq_scales, sdt, "xq_scales", (M // 16, K // 16), used=gemm)
    _need(rq_codes, torch.uint8, "rq_codes", (N, K // 2), used=gemm)
    _need(rq_scales, sdt, "rq_scales", (N // 16, K // 16), used=gemm)
    _need(T, torch.float32, "T", (M, rs + r))
    dev = T.device
    if out is None:
        out = (torch.empty((M, N), dtype=torch.bfloat16, device=dev), torch.empty((M, N), dtype=torch.bfloat16, device=dev),
               torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
               torch.empty((M // 16, N // 16), dtype=torch.uint8, device=dev))
    Y, H, hc, hs = out
    _need(Y, torch.bfloat16, "Y", (M, N))
    _need(H, torch.bfloat16, "H", (M, N))
    _need(hc, torch.uint8, "h_codes", (M, N // 2))
    _need(hs, torch.uint8, "h_scales", (M // 16, N // 16))
    _same_device(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, Y, H, hc, hs)
    st = lib().ft_linear_fwd_gelu(M, N, K, _MODES[mode], xq_codes.data_ptr(), xq_scales.data_ptr(),
                                  rq_codes.data_ptr(), rq_scales.data_ptr(), T.data_ptr(),
                                  L2.data_ptr(), rs, B.data_ptr(), r, Y.data_ptr(), H.data_ptr(),
                                  hc.data_ptr(), hs.data_ptr(), _stream(T))
    check("ft_linear_fwd_gelu", st)
    return Y, H, hc, hs


def linear_bwd_workspace(M: int, N: int, K: int, r: int) -> int:
    return int(lib().ft_linear_bwd_workspace(M, N, K, r))


def linear_bwd_plan(M: int, N: int, K: int, r: int, with_db: bool = True):
    """(tile_m, tile_n, gemm_splits, adapter_workgroups, adapter_splits) of
    ft_linear_bwd (adapter_workgroups 0: the adapter gradients on the side stream)."""
    import ctypes
    out = (ctypes.c_int32 * 5)()
    check("ft_linear_bwd_plan", lib().ft_linear_bwd_plan(M, N, K, r, int(with_db), ctypes.addressof(out)))
    return tuple(int(v) for v in out)


def _bwd_common(V, L1t, At, X, G, T, M, N, K, dX, dAt, dB, out_dtype, x_name="X", g_name="G"):
    """Shared checks and output allocation of the backward calls: returns (rs, r, dX, dAt, dB)."""
    rs, r = _up_factors(L1t, At, K, names=("L1t", "At"))
    rho = rs + r
    dev = V.device if isinstance(V, torch.Tensor) else None
    _need(V, torch.float32, "V", (M, rho))
    _need(T, torch.float32, "T", (M, rho))
    if X is not None:
        _need(X, torch.bfloat16, x_name, (M, K))
    if G is not None:
        _need(G, torch.bfloat16, g_name, (M, N))
    if dX is None:
        dX = torch.empty((M, K), dtype=out_dtype, device=dev)
    if dAt is None:
        dAt = torch.empty((r, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    _out_dtype(dX, "dX")
    _need(dX, dX.dtype, "dX", (M, K))
    _need(dAt, torch.float32, "dAt", (r, K))
    _need(dB, torch.float32, "dB", (r, N))
    return rs, r, dX, dAt, dB


def linear_bwd(gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, At, X, G, T,
               M: int, N: int, K: int, out_dtype=torch.float32, mode: str = "pow2",
               workspace: Optional[torch.Tensor] = None, dX: Optional[torch.Tensor] = None,
               dAt: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None, prepare: bool = False,
               skip_dB: bool = False):
    """dX, dAt, dB of Eq. 3 and section 3.2 (see include/ft.h; ``prepare``: return a ``Prepared`` call).
    ``skip_dB``: dB is not computed (it was taken in the pass over G by quant_lowrank_db); dB is returned as None."""
    _mult16("linear_bwd", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    sdt = _sdt(mode)
    rs, r, dX, dAt, dB = _bwd_common(V, L1t, At, X, G, T, M, N, K, dX, dAt, dB, out_dtype)
    _need(gq_codes, torch.uint8, "gq_codes", (M, N // 2), used=gemm)
    _need(gq_scales, sdt, "gq_scales", (M // 16, N // 16), used=gemm)
    _need(rq_codes_cm, torch.uint8, "rq_codes_cm", (K, N // 2), used=gemm)
    _need(rq_scales_cm, sdt, "rq_scales_cm", (K // 16, N // 16), used=gemm)
    workspace = _ws(workspace, linear_bwd_workspace(M, N, K, r), V.device)
    _same_device(gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, At, X, G, T, dX, dAt, dB, workspace)
    args = (M, N, K, _MODES[mode], gq_codes.data_ptr(), gq_scales.data_ptr(), rq_codes_cm.data_ptr(),
            rq_scales_cm.data_ptr(), V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r, X.data_ptr(), G.data_ptr(),
            T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype], dAt.data_ptr(), None if skip_dB else dB.data_ptr(),
            workspace.data_ptr(), workspace.numel())
    return _issue("ft_linear_bwd", args, V.device, (dX, dAt, None if skip_dB else dB),
                  (gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, At, X, G, T, dX, dAt, dB, workspace),
                  prepare)


def linear_fwd_op(x_op, x_op_scales, r_op, r_op_scales, T, L2, B, M: int, N: int, K: int,
                  out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """Y of Eq. 2 from pair-merged operands (ft_quant_block16_op op_rm of X and of R)."""
    _mult16("linear_fwd_op", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r = _up_factors(L2, B, N)
    (xa, xb), (xc, xd) = operand_shapes(M, K)
    (ra_, rb_), (rc, rd) = operand_shapes(N, K)
    _need(x_op, torch.uint8, "x_op", (xa, xb), used=gemm)
    _need(x_op_scales, torch.uint8, "x_op_scales", (xc, xd), used=gemm)
    _need(r_op, torch.uint8, "r_op", (ra_, rb_), used=gemm)
    _need(r_op_scales, torch.uint8, "r_op_scales", (rc, rd), used=gemm)
    _need(T, torch.float32, "T", (M, rs + r))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    odt = _out_dtype(out, "out")
    _need(out, out.dtype, "out", (M, N))
    _same_device(x_op, x_op_scales, r_op, r_op_scales, T, L2, B, out)
    st = lib().ft_linear_fwd_op(M, N, K, x_op.data_ptr(), x_op_scales.data_ptr(), r_op.data_ptr(),
                                r_op_scales.data_ptr(), T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r,
                                out.data_ptr(), odt, _stream(T))
    check("ft_linear_fwd_op", st)
    return out


def linear_bwd_op(g_op, g_op_scales, rt_op, rt_op_scales, V, L1t, At, X, G, T, M: int, N: int, K: int,
                  out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                  dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                  dB: Optional[torch.Tensor] = None):
    """dX, dAt, dB of Eq. 3 from pair-merged operands (op_rm of G, op_cm of R)."""
    _mult16("linear_bwd_op", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r, dX, dAt, dB = _bwd_common(V, L1t, At, X, G, T, M, N, K, dX, dAt, dB, out_dtype)
    (ga, gb), (gc, gd) = operand_shapes(M, N)
    (ta, tb), (tc, td) = operand_shapes(K, N)
    _need(g_op, torch.uint8, "g_op", (ga, gb), used=gemm)
    _need(g_op_scales, torch.uint8, "g_op_scales", (gc, gd), used=gemm)
    _need(rt_op, torch.uint8, "rt_op", (ta, tb), used=gemm)
    _need(rt_op_scales, torch.uint8, "rt_op_scales", (tc, td), used=gemm)
    workspace = _ws(workspace, linear_bwd_workspace(M, N, K, r), V.device)
    _same_device(g_op, g_op_scales, rt_op, rt_op_scales, V, L1t, At, X, G, T, dX, dAt, dB, workspace)
    st = lib().ft_linear_bwd_op(M, N, K, g_op.data_ptr(), g_op_scales.data_ptr(), rt_op.data_ptr(),
                                rt_op_scales.data_ptr(), V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r,
                                X.data_ptr(), G.data_ptr(), T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype],
                                dAt.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream(V))
    check("ft_linear_bwd_op", st)
    return dX, dAt, dB


def linear_fwd_a16(X, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """W4A16 forward: Y = X deq(Rq)^T + T[:, :rs] L2 + T[:, rs:] B (X bf16, unquantized)."""
    _mult16("linear_fwd_a16", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r = _up_factors(L2, B, N)
    _need(X, torch.bfloat16, "X", (M, K))
    _need(rq_codes, torch.uint8, "rq_codes", (N, K // 2), used=gemm)
    _need(rq_scales, torch.uint8, "rq_scales", (N // 16, K // 16), used=gemm)
    _need(T, torch.float32, "T", (M, rs + r))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    odt = _out_dtype(out, "out")
    _need(out, out.dtype, "out", (M, N))
    _same_device(X, rq_codes, rq_scales, T, L2, B, out)
    st = lib().ft_linear_fwd_a16(M, N, K, X.data_ptr(), rq_codes.data_ptr(), rq_scales.data_ptr(),
                                 T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r, out.data_ptr(),
                                 odt, _stream(X))
    check("ft_linear_fwd_a16", st)
    return out


def linear_bwd_g16(G, rq_codes_cm, rq_scales_cm, V, L1t, At, X, T, M: int, N: int, K: int,
                   out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                   dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                   dB: Optional[torch.Tensor] = None):
    """G16 backward: dX = G deq(Rq) + V [L1^T; A^T] (G bf16, unquantized) and dAt, dB."""
    _mult16("linear_bwd_g16", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r, dX, dAt, dB = _bwd_common(V, L1t, At, X, G, T, M, N, K, dX, dAt, dB, out_dtype)
    _need(rq_codes_cm, torch.uint8, "rq_codes_cm", (K, N // 2), used=gemm)
    _need(rq_scales_cm, torch.uint8, "rq_scales_cm", (K // 16, N // 16), used=gemm)
    workspace = _ws(workspace, linear_bwd_workspace(M, N, K, r), G.device)
    _same_device(G, rq_codes_cm, rq_scales_cm, V, L1t, At, X, T, dX, dAt, dB, workspace)
    st = lib().ft_linear_bwd_g16(M, N, K, G.data_ptr(), rq_codes_cm.data_ptr(), rq_scales_cm.data_ptr(),
                                 V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r, X.data_ptr(),
                                 T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype], dAt.data_ptr(),
                                 dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(G))
    check("ft_linear_bwd_g16", st)
    return dX, dAt, dB


def _group(group: int) -> None:
    if group not in (16, 32):
        raise ValueError(f"group must be 16 or 32, got {group}")


def quant_group(x: torch.Tensor, group: int, out=None):
    """Q(x) in 1 x group groups along rows: (codes [rows, cols/2], scales [rows, cols/group])."""
    _group(group)
    _need_matrix(x, "x")
    rows, cols = x.shape
    _mult16("quant_group", rows, cols)
    if cols % group:
        raise ValueError(f"cols {cols} is not a multiple of the group {group}")
    if out is None:
        out = (torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device),
               torch.empty((rows, cols // group), dtype=torch.uint8, device=x.device))
    codes, scales = out
    _need(codes, torch.uint8, "codes", (rows, cols // 2))
    _need(scales, torch.uint8, "scales", (rows, cols // group))
    _same_device(x, codes, scales)
    st = lib().ft_quant_group(x.data_ptr(), rows, cols, x.stride(0), group, codes.data_ptr(), scales.data_ptr(),
                              _stream(x))
    check("ft_quant_group", st)
    return codes, scales


def requant_group_t(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int, group: int, out=None):
    """Q(deq(Q(R))^T) in 1 x group groups: (codes_t [cols, rows/2], scales_t [cols, rows/group])."""
    _group(group)
    _mult16("requant_group_t", rows, cols)
    if rows % group or cols % group:
        raise ValueError(f"rows and cols must be multiples of the group {group}")
    _need(codes, torch.uint8, "codes", (rows, cols // 2))
    _need(scales, torch.uint8, "scales", (rows, cols // group))
    if out is None:
        out = (torch.empty((cols, rows // 2), dtype=torch.uint8, device=codes.device),
               torch.empty((cols, rows // group), dtype=torch.uint8, device=codes.device))
    ct, st_ = out
    _need(ct, torch.uint8, "codes_t", (cols, rows // 2))
    _need(st_, torch.uint8, "scales_t", (cols, rows // group))
    _same_device(codes, scales, ct, st_)
    st = lib().ft_requant_group_t(codes.data_ptr(), scales.data_ptr(), rows, cols, group, ct.data_ptr(),
                                  st_.data_ptr(), _stream(codes))
    check("ft_requant_group_t", st)
    return ct, st_


def linear_fwd_grp(group, xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """Eq. 2 with 1 x group scaled operands (ft_quant_group of X and R)."""
    _group(group)
    _mult16("linear_fwd_grp", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r = _up_factors(L2, B, N)
    _need(xq_codes, torch.uint8, "xq_codes", (M, K // 2), used=gemm)
    _need(xq_scales, torch.uint8, "xq_scales", (M, K // group), used=gemm)
    _need(rq_codes, torch.uint8, "rq_codes", (N, K // 2), used=gemm)
    _need(rq_scales, torch.uint8, "rq_scales", (N, K // group), used=gemm)
    _need(T, torch.float32, "T", (M, rs + r))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    odt = _out_dtype(out, "out")
    _need(out, out.dtype, "out", (M, N))
    _same_device(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, out)
    st = lib().ft_linear_fwd_grp(M, N, K, group, xq_codes.data_ptr(), xq_scales.data_ptr(), rq_codes.data_ptr(),
                                 rq_scales.data_ptr(), T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r,
                                 out.data_ptr(), odt, _stream(T))
    check("ft_linear_fwd_grp", st)
    return out


def linear_bwd_grp(group, gq_codes, gq_scales, rtq_codes, rtq_scales, V, L1t, At, X, G, T, M: int, N: int, K: int,
                   out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                   dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                   dB: Optional[torch.Tensor] = None):
    """Eq. 3 and the adapter gradients with 1 x group scaled operands (rtq: ft_requant_group_t of Q(R))."""
    _group(group)
    _mult16("linear_bwd_grp", M, N, K)
    gemm = M > 0 and N > 0 and K > 0
    rs, r, dX, dAt, dB = _bwd_common(V, L1t, At, X, G, T, M, N, K, dX, dAt, dB, out_dtype)
    _need(gq_codes, torch.uint8, "gq_codes", (M, N // 2), used=gemm)
    _need(gq_scales, torch.uint8, "gq_scales", (M, N // group), used=gemm)
    _need(rtq_codes, torch.uint8, "rtq_codes", (K, N // 2), used=gemm)
    _need(rtq_scales, torch.uint8, "rtq_scales", (K, N // group), used=gemm)
    workspace = _ws(workspace, linear_bwd_workspace(M, N, K, r), V.device)
    _same_device(gq_codes, gq_scales, rtq_codes, rtq_scales, V, L1t, At, X, G, T, dX, dAt, dB, workspace)
    st = lib().ft_linear_bwd_grp(M, N, K, group, gq_codes.data_ptr(), gq_scales.data_ptr(), rtq_codes.data_ptr(),
                                 rtq_scales.data_ptr(), V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r,
                                 X.data_ptr(), G.data_ptr(), T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype],
                                 dAt.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(V))
    check("ft_linear_bwd_grp", st)
    return dX, dAt, dB


def stream_2to1(x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Measurement reference: out[i] = high byte of the 16-bit x[i] (2 bytes read,
    1 written per element; see ft_stream_2to1)."""
    if x.element_size() != 2:
        raise ValueError("x must hold 16-bit elements")
    _need(x, x.dtype, "x")
    _need(out, torch.uint8, "out", min_numel=x.numel())
    _same_device(x, out)
    check("ft_stream_2to1", lib().ft_stream_2to1(x.data_ptr(), x.numel(), out.data_ptr(), _stream(x)))
    return out


def gelu_fwd(y: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(y, torch.bfloat16, "y")
    if out is None:
        out = torch.empty_like(y)
    _need(out, torch.bfloat16, "out", tuple(y.shape))
    _same_device(y, out)
    st = lib().ft_gelu_fwd(y.data_ptr(), y.numel(), out.data_ptr(), _stream(y))
    check("ft_gelu_fwd", st)
    return out


def gelu_bwd(y: torch.Tensor, dh: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(y, torch.bfloat16, "y")
    _need(dh, torch.bfloat16, "dh", tuple(y.shape))
    if out is None:
        out = torch.empty_like(y)
    _need(out, torch.bfloat16, "out", tuple(y.shape))
    _same_device(y, dh, out)
    st = lib().ft_gelu_bwd(y.data_ptr(), dh.data_ptr(), y.numel(), out.data_ptr(), _stream(y))
    check("ft_gelu_bwd", st)
    return out
