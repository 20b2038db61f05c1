"""ft_linear_bwd_noalloc (the backward for callers that cannot allocate) against
ft_linear_bwd through the C ABI: identical dX, dA, dB bits, on two calls in a
row (the second smaller, so it runs on the first call's leftover scratch)."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _prepared(M, K, N, rs, r, seed):
    import torch
    from bit_quantized_lora_amd import ops
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_dist="t3", x_outlier_count=4, x_outlier_mult=30.0)
    d = synth.make_linear(spec, np.random.default_rng(seed))
    X, R, G = dev_bf16(d["X"]), dev_bf16(d["R"]), dev_bf16(d["G"])
    L1t, At = dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(np.ascontiguousarray(d["A"].T))
    L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
    _, rqc, _, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
    T, _, _ = ops.quant_lowrank(X, L1t, At)
    V, gq, gs = ops.quant_lowrank(G, L2, B)
    torch.cuda.synchronize()
    return dict(M=M, K=K, N=N, rs=rs, r=r, X=X, G=G, L1t=L1t, At=At, rqc=rqc, rsct=rsct, T=T, V=V, gq=gq, gs=gs)


def _noalloc(p, dx_dtype):
    import torch
    from bit_quantized_lora_amd import _lib
    L = _lib.lib()
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    dX = torch.empty((M, K), dtype=dx_dtype, device="cuda")
    dAt = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((r, N), dtype=torch.float32, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.ft_linear_bwd_noalloc(M, N, K, _lib.FT_SCALE_POW2, ptr(p["gq"]), ptr(p["gs"]), ptr(p["rqc"]),
                                 ptr(p["rsct"]), ptr(p["V"]), ptr(p["L1t"]), p["rs"], ptr(p["At"]), r,
                                 ptr(p["X"]), ptr(p["G"]), ptr(p["T"]), ptr(dX),
                                 _lib.FT_OUT_BF16 if dx_dtype == torch.bfloat16 else _lib.FT_OUT_F32,
                                 ptr(dAt), ptr(dB), torch.cuda.current_stream().cuda_stream)
    _lib.check("ft_linear_bwd_noalloc", st)
    return dX, dAt, dB


def test_noalloc_backward_matches_the_workspace_backward():
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    for (M, K, N, rs, r), dt in (((4608, 3072, 3072, 32, 32), torch.bfloat16), ((272, 384, 528, 16, 16), torch.float32)):
        say(f"[noalloc] M={M} K={K} N={N} rs={rs} r={r} dX {dt}")
        p = _prepared(M, K, N, rs, r, M + K + N)
        got = _noalloc(p, dt)
        ref = ops.linear_bwd(p["gq"], p["gs"], p["rqc"], p["rsct"], p["V"], p["L1t"], p["At"], p["X"], p["G"],
                             p["T"], M, N, K, out_dtype=dt)
        torch.cuda.synchronize()
        for name, a, b in zip(("dX", "dAt", "dB"), got, ref):
            ha, hb = host(a), host(b)
            assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), f"{name} differs"
        say(f"[noalloc]   dX, dAt, dB bit-identical to ft_linear_bwd")
