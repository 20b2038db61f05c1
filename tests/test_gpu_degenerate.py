"""Degenerate sizes on the GPU: an empty reduction (K = 0 forward, N = 0
backward) leaves only the low-rank terms of Eq. 2 and Eq. 3, and zero tokens
(M = 0) make the adapter gradients of section 3.2 empty sums (zeros).  Every
GEMM entry point is run; results against fp64 products of the same inputs."""
import numpy as np
import pytest

import oracle as O
from gpu_util import host, require_gpu, say

pytestmark = pytest.mark.gpu

FWD_PATHS = ["codes", "op", "a16", "grp16", "grp32"]
BWD_PATHS = ["codes", "op", "g16", "grp16", "grp32"]


def _t(torch, shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (scale * torch.randn(shape, device="cuda", generator=g)).to(dtype)


@pytest.mark.parametrize("path", FWD_PATHS)
def test_forward_empty_reduction(path):
    """K = 0: Y = T[:, :rs] L2 + T[:, rs:] B (the GEMM reads no operand)."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, N, K, rs, r = 48, 272, 0, 16, 32
    T = _t(torch, (M, rs + r), torch.float32, 1)
    L2 = _t(torch, (rs, N), torch.bfloat16, 2, 0.1)
    B = _t(torch, (r, N), torch.bfloat16, 3, 0.1)
    e8 = torch.empty((0,), dtype=torch.uint8, device="cuda")
    say(f"[degenerate] forward K=0 path={path}")
    if path == "codes":
        Y = ops.linear_fwd(e8, e8, e8, e8, T, L2, B, M, N, K)
    elif path == "op":
        Y = ops.linear_fwd_op(e8, e8, e8, e8, T, L2, B, M, N, K)
    elif path == "a16":
        Y = ops.linear_fwd_a16(torch.empty((0,), dtype=torch.bfloat16, device="cuda"), e8, e8, T, L2, B, M, N, K)
    else:
        Y = ops.linear_fwd_grp(int(path[3:]), e8, e8, e8, e8, T, L2, B, M, N, K)
    W = np.concatenate([host(L2).view(np.uint16), host(B).view(np.uint16)])
    ref = host(T).astype(np.float64) @ O.bf16_to_f64(W)
    assert O.rel_frob(host(Y).astype(np.float64), ref) < 1e-4


@pytest.mark.parametrize("path", BWD_PATHS)
def test_backward_empty_reduction(path):
    """N = 0: dX = V[:, :rs] L1t + V[:, rs:] At, dAt = V[:, rs:]^T X, dB empty."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, N, K, rs, r = 48, 0, 144, 16, 16
    V = _t(torch, (M, rs + r), torch.float32, 4)
    T = _t(torch, (M, rs + r), torch.float32, 5)
    L1t = _t(torch, (rs, K), torch.bfloat16, 6, 0.1)
    At = _t(torch, (r, K), torch.bfloat16, 7, 0.1)
    X = _t(torch, (M, K), torch.bfloat16, 8)
    e8 = torch.empty((0,), dtype=torch.uint8, device="cuda")
    eb = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    say(f"[degenerate] backward N=0 path={path}")
    if path == "codes":
        dX, dAt, dB = ops.linear_bwd(e8, e8, e8, e8, V, L1t, At, X, eb, T, M, N, K)
    elif path == "op":
        dX, dAt, dB = ops.linear_bwd_op(e8, e8, e8, e8, V, L1t, At, X, eb, T, M, N, K)
    elif path == "g16":
        dX, dAt, dB = ops.linear_bwd_g16(eb, e8, e8, V, L1t, At, X, T, M, N, K)
    else:
        dX, dAt, dB = ops.linear_bwd_grp(int(path[3:]), e8, e8, e8, e8, V, L1t, At, X, eb, T, M, N, K)
    Vh = host(V).astype(np.float64)
    W = np.concatenate([host(L1t).view(np.uint16), host(At).view(np.uint16)])
    assert O.rel_frob(host(dX).astype(np.float64), Vh @ O.bf16_to_f64(W)) < 1e-4
    ref_dAt = Vh[:, rs:].T @ O.bf16_to_f64(host(X).view(np.uint16))
    assert O.rel_frob(host(dAt).astype(np.float64), ref_dAt) < 1e-4
    assert dB.numel() == 0


@pytest.mark.parametrize("path", BWD_PATHS)
def test_backward_zero_tokens(path):
    """M = 0: the adapter gradients are sums over no tokens, so exactly zero
    (outputs pre-filled with NaN to see that they are written)."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, N, K, rs, r = 0, 256, 128, 16, 16
    e8 = torch.empty((0,), dtype=torch.uint8, device="cuda")
    V = torch.empty((0, rs + r), dtype=torch.float32, device="cuda")
    T = torch.empty((0, rs + r), dtype=torch.float32, device="cuda")
    X = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    L1t = _t(torch, (rs, K), torch.bfloat16, 9)
    At = _t(torch, (r, K), torch.bfloat16, 10)
    dAt = torch.full((r, K), float("nan"), device="cuda")
    dB = torch.full((r, N), float("nan"), device="cuda")
    dX = torch.empty((0, K), dtype=torch.float32, device="cuda")
    say(f"[degenerate] backward M=0 path={path}")
    if path == "codes":
        ops.linear_bwd(e8, e8, e8, e8, V, L1t, At, X, G, T, M, N, K, dX=dX, dAt=dAt, dB=dB)
    elif path == "op":
        ops.linear_bwd_op(e8, e8, e8, e8, V, L1t, At, X, G, T, M, N, K, dX=dX, dAt=dAt, dB=dB)
    elif path == "g16":
        ops.linear_bwd_g16(G, e8, e8, V, L1t, At, X, T, M, N, K, dX=dX, dAt=dAt, dB=dB)
    else:
        ops.linear_bwd_grp(int(path[3:]), e8, e8, e8, e8, V, L1t, At, X, G, T, M, N, K, dX=dX, dAt=dAt, dB=dB)
    assert np.all(host(dAt) == 0.0) and np.all(host(dB) == 0.0)
