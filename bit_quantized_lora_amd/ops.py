"""Thin torch binding of the ft C ABI (argument marshalling only).

Each function takes CUDA (HIP) tensors, allocates outputs with torch (device
memory is torch's job here), passes raw pointers and the current stream to
libft.so and raises ``FtError`` on a non-OK status.  No arithmetic of the
method happens in Python.
"""
from __future__ import annotations

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


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def quant_block16(x: torch.Tensor, mode: str = "pow2", rm: bool = True, cm: bool = False,
                  out: Optional[Tuple] = None, scales_cm: bool = False):
    """Q(x) for a bf16 [rows, cols] matrix -> (codes_rm, codes_cm, scales), plus
    the transposed scale grid as a fourth element when ``scales_cm`` is set.

    ``out`` may supply preallocated (codes_rm, codes_cm, scales[, scales_cm]) buffers.
    """
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D matrix with unit column stride")
    rows, cols = x.shape
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
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D matrix with unit column stride")
    rows, cols = x.shape
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
    g = lambda k: _ptr(out.get(k))
    st = lib().ft_quant_block16_op(x.data_ptr(), rows, cols, x.stride(0), g("codes_rm"), g("codes_cm"),
                                   g("scales"), g("scales_cm"), g("op_rm"), g("op_rm_scales"), g("op_cm"),
                                   g("op_cm_scales"), _stream(x))
    check("ft_quant_block16_op", st)
    return out


def lowrank_workspace(M: int, Kin: int, rho: int) -> int:
    return int(lib().ft_lowrank_workspace(M, Kin, rho))


def lowrank_fused(inp: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = [inp wa^T | inp wb^T] in fp32; wa [ra, Kin], wb [rb, Kin] bf16."""
    _need(inp, torch.bfloat16, "inp")
    M, Kin = inp.shape
    ra, rb = wa.shape[0], wb.shape[0]
    for w, n in ((wa, "wa"), (wb, "wb")):
        _need(w, torch.bfloat16, n)
        if w.dim() != 2 or w.shape[1] != Kin or not w.is_contiguous():
            raise ValueError(f"{n} must be contiguous [rank, {Kin}]")
    if out is None:
        out = torch.empty((M, ra + rb), dtype=torch.float32, device=inp.device)
    ws_bytes = lowrank_workspace(M, Kin, ra + rb)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=inp.device)
    st = lib().ft_lowrank_fused(inp.data_ptr(), M, Kin, inp.stride(0), wa.data_ptr(), ra,
                                wb.data_ptr(), rb, out.data_ptr(), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(inp))
    check("ft_lowrank_fused", st)
    return out


def quant_lowrank(inp: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor, out: Optional[torch.Tensor] = None,
                  codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """(out, codes_rm, scales): [inp wa^T | inp wb^T] and Q(inp) in one read of inp."""
    _need(inp, torch.bfloat16, "inp")
    M, Kin = inp.shape
    ra, rb = wa.shape[0], wb.shape[0]
    dev = inp.device
    if out is None:
        out = torch.empty((M, ra + rb), dtype=torch.float32, device=dev)
    if codes is None:
        codes = torch.empty((M, Kin // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M // 16, Kin // 16), dtype=torch.uint8, device=dev)
    ws_bytes = lowrank_workspace(M, Kin, ra + rb)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    st = lib().ft_quant_lowrank(inp.data_ptr(), M, Kin, inp.stride(0), wa.data_ptr(), ra, wb.data_ptr(), rb,
                                out.data_ptr(), codes.data_ptr(), scales.data_ptr(), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(inp))
    check("ft_quant_lowrank", st)
    return out, codes, scales


def gelu_quant_lowrank(y: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor, out=None, workspace=None):
    """h = GELU(y), Q(h) and [h wa^T | h wb^T] from one read of y:
    returns (h, T, codes, scales)."""
    _need(y, torch.bfloat16, "y")
    M, Kin = y.shape
    ra, rb = wa.shape[0], wb.shape[0]
    dev = y.device
    if out is None:
        out = (torch.empty((M, Kin), dtype=torch.bfloat16, device=dev),
               torch.empty((M, ra + rb), dtype=torch.float32, device=dev),
               torch.empty((M, Kin // 2), dtype=torch.uint8, device=dev),
               torch.empty((M // 16, Kin // 16), dtype=torch.uint8, device=dev))
    h, T, codes, scales = out
    nb = lowrank_workspace(M, Kin, ra + rb)
    if workspace is None or workspace.numel() < nb:
        workspace = torch.empty((max(nb, 16),), dtype=torch.uint8, device=dev)
    st = lib().ft_gelu_quant_lowrank(y.data_ptr(), M, Kin, wa.data_ptr(), ra, wb.data_ptr(), rb, h.data_ptr(),
                                     T.data_ptr(), codes.data_ptr(), scales.data_ptr(), workspace.data_ptr(),
                                     workspace.numel(), _stream(y))
    check("ft_gelu_quant_lowrank", st)
    return h, T, codes, scales


def linear_fwd(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
               out_dtype=torch.float32, mode: str = "pow2", out: Optional[torch.Tensor] = None):
    """Y = deq(Xq) deq(Rq)^T + T[:, :rs] L2 + T[:, rs:] B."""
    rs, r = L2.shape[0], B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    st = lib().ft_linear_fwd(M, N, K, _MODES[mode], xq_codes.data_ptr(), xq_scales.data_ptr(),
                             rq_codes.data_ptr(), rq_scales.data_ptr(), T.data_ptr(),
                             L2.data_ptr(), rs, B.data_ptr(), r, out.data_ptr(), _OUT[out.dtype],
                             _stream(T))
    check("ft_linear_fwd", st)
    return out


def linear_fwd_gelu(xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
                    mode: str = "pow2", out=None):
    """First linear of an MLP with the fused epilogue: Y (bf16), H = GELU(Y) (bf16)
    and Q(H) (row-major codes, scales); returns (Y, H, h_codes, h_scales)."""
    rs, r = L2.shape[0], B.shape[0]
    dev = T.device
    if out is None:
        out = (torch.empty((M, N), dtype=torch.bfloat16, device=dev), torch.empty((M, N), dtype=torch.bfloat16, device=dev),
               torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
               torch.empty((M // 16, N // 16), dtype=torch.uint8, device=dev))
    Y, H, hc, hs = out
    st = lib().ft_linear_fwd_gelu(M, N, K, _MODES[mode], xq_codes.data_ptr(), xq_scales.data_ptr(),
                                  rq_codes.data_ptr(), rq_scales.data_ptr(), T.data_ptr(),
                                  L2.data_ptr(), rs, B.data_ptr(), r, Y.data_ptr(), H.data_ptr(),
                                  hc.data_ptr(), hs.data_ptr(), _stream(T))
    check("ft_linear_fwd_gelu", st)
    return Y, H, hc, hs


def linear_bwd_workspace(M: int, N: int, K: int, r: int) -> int:
    return int(lib().ft_linear_bwd_workspace(M, N, K, r))


def linear_bwd(gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, At, X, G, T,
               M: int, N: int, K: int, out_dtype=torch.float32, mode: str = "pow2",
               workspace: Optional[torch.Tensor] = None, dX: Optional[torch.Tensor] = None,
               dAt: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None):
    """dX, dAt, dB of Eq. 3 and section 3.2 (see include/ft.h)."""
    rs, r = L1t.shape[0], At.shape[0]
    dev = V.device
    if dX is None:
        dX = torch.empty((M, K), dtype=out_dtype, device=dev)
    if dAt is None:
        dAt = torch.empty((r, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    ws_bytes = linear_bwd_workspace(M, N, K, r)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    st = lib().ft_linear_bwd(M, N, K, _MODES[mode], gq_codes.data_ptr(), gq_scales.data_ptr(),
                             rq_codes_cm.data_ptr(), rq_scales_cm.data_ptr(), V.data_ptr(),
                             L1t.data_ptr(), rs, At.data_ptr(), r, X.data_ptr(), G.data_ptr(),
                             T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype], dAt.data_ptr(),
                             dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(V))
    check("ft_linear_bwd", st)
    return dX, dAt, dB


def linear_fwd_op(x_op, x_op_scales, r_op, r_op_scales, T, L2, B, M: int, N: int, K: int,
                  out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """Y of Eq. 2 from pair-merged operands (ft_quant_block16_op op_rm of X and of R)."""
    rs, r = L2.shape[0], B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    st = lib().ft_linear_fwd_op(M, N, K, x_op.data_ptr(), x_op_scales.data_ptr(), r_op.data_ptr(),
                                r_op_scales.data_ptr(), T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r,
                                out.data_ptr(), _OUT[out.dtype], _stream(T))
    check("ft_linear_fwd_op", st)
    return out


def linear_bwd_op(g_op, g_op_scales, rt_op, rt_op_scales, V, L1t, At, X, G, T, M: int, N: int, K: int,
                  out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                  dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                  dB: Optional[torch.Tensor] = None):
    """dX, dAt, dB of Eq. 3 from pair-merged operands (op_rm of G, op_cm of R)."""
    rs, r = L1t.shape[0], At.shape[0]
    dev = V.device
    if dX is None:
        dX = torch.empty((M, K), dtype=out_dtype, device=dev)
    if dAt is None:
        dAt = torch.empty((r, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    ws_bytes = linear_bwd_workspace(M, N, K, r)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
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
    rs, r = L2.shape[0], B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    st = lib().ft_linear_fwd_a16(M, N, K, X.data_ptr(), rq_codes.data_ptr(), rq_scales.data_ptr(),
                                 T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r, out.data_ptr(),
                                 _OUT[out.dtype], _stream(X))
    check("ft_linear_fwd_a16", st)
    return out


def linear_bwd_g16(G, rq_codes_cm, rq_scales_cm, V, L1t, At, X, T, M: int, N: int, K: int,
                   out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                   dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                   dB: Optional[torch.Tensor] = None):
    """G16 backward: dX = G deq(Rq) + V [L1^T; A^T] (G bf16, unquantized) and dAt, dB."""
    rs, r = L1t.shape[0], At.shape[0]
    dev = G.device
    if dX is None:
        dX = torch.empty((M, K), dtype=out_dtype, device=dev)
    if dAt is None:
        dAt = torch.empty((r, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    ws_bytes = linear_bwd_workspace(M, N, K, r)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    st = lib().ft_linear_bwd_g16(M, N, K, G.data_ptr(), rq_codes_cm.data_ptr(), rq_scales_cm.data_ptr(),
                                 V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r, X.data_ptr(),
                                 T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype], dAt.data_ptr(),
                                 dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(G))
    check("ft_linear_bwd_g16", st)
    return dX, dAt, dB


def quant_group(x: torch.Tensor, group: int, out=None):
    """Q(x) in 1 x group groups along rows: (codes [rows, cols/2], scales [rows, cols/group])."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if out is None:
        out = (torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device),
               torch.empty((rows, cols // group), dtype=torch.uint8, device=x.device))
    codes, scales = out
    st = lib().ft_quant_group(x.data_ptr(), rows, cols, x.stride(0), group, codes.data_ptr(), scales.data_ptr(),
                              _stream(x))
    check("ft_quant_group", st)
    return codes, scales


def requant_group_t(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int, group: int, out=None):
    """Q(deq(Q(R))^T) in 1 x group groups: (codes_t [cols, rows/2], scales_t [cols, rows/group])."""
    if out is None:
        out = (torch.empty((cols, rows // 2), dtype=torch.uint8, device=codes.device),
               torch.empty((cols, rows // group), dtype=torch.uint8, device=codes.device))
    ct, st_ = out
    st = lib().ft_requant_group_t(codes.data_ptr(), scales.data_ptr(), rows, cols, group, ct.data_ptr(),
                                  st_.data_ptr(), _stream(codes))
    check("ft_requant_group_t", st)
    return ct, st_


def linear_fwd_grp(group, xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B, M: int, N: int, K: int,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """Eq. 2 with 1 x group scaled operands (ft_quant_group of X and R)."""
    rs, r = L2.shape[0], B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=T.device)
    st = lib().ft_linear_fwd_grp(M, N, K, group, xq_codes.data_ptr(), xq_scales.data_ptr(), rq_codes.data_ptr(),
                                 rq_scales.data_ptr(), T.data_ptr(), L2.data_ptr(), rs, B.data_ptr(), r,
                                 out.data_ptr(), _OUT[out.dtype], _stream(T))
    check("ft_linear_fwd_grp", st)
    return out


def linear_bwd_grp(group, gq_codes, gq_scales, rtq_codes, rtq_scales, V, L1t, At, X, G, T, M: int, N: int, K: int,
                   out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                   dX: Optional[torch.Tensor] = None, dAt: Optional[torch.Tensor] = None,
                   dB: Optional[torch.Tensor] = None):
    """Eq. 3 and the adapter gradients with 1 x group scaled operands (rtq: ft_requant_group_t of Q(R))."""
    rs, r = L1t.shape[0], At.shape[0]
    dev = V.device
    if dX is None:
        dX = torch.empty((M, K), dtype=out_dtype, device=dev)
    if dAt is None:
        dAt = torch.empty((r, K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    ws_bytes = linear_bwd_workspace(M, N, K, r)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    st = lib().ft_linear_bwd_grp(M, N, K, group, gq_codes.data_ptr(), gq_scales.data_ptr(), rtq_codes.data_ptr(),
                                 rtq_scales.data_ptr(), V.data_ptr(), L1t.data_ptr(), rs, At.data_ptr(), r,
                                 X.data_ptr(), G.data_ptr(), T.data_ptr(), dX.data_ptr(), _OUT[dX.dtype],
                                 dAt.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(V))
    check("ft_linear_bwd_grp", st)
    return dX, dAt, dB


def gelu_fwd(y: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(y, torch.bfloat16, "y")
    if out is None:
        out = torch.empty_like(y)
    st = lib().ft_gelu_fwd(y.data_ptr(), y.numel(), out.data_ptr(), _stream(y))
    check("ft_gelu_fwd", st)
    return out


def gelu_bwd(y: torch.Tensor, dh: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(y, torch.bfloat16, "y"); _need(dh, torch.bfloat16, "dh")
    if out is None:
        out = torch.empty_like(y)
    st = lib().ft_gelu_bwd(y.data_ptr(), dh.data_ptr(), y.numel(), out.data_ptr(), _stream(y))
    check("ft_gelu_bwd", st)
    return out
