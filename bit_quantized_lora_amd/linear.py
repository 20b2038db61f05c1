"""The triple-branch W4A4G4 linear as a torch module (FourTune section 3.1,
Eq. 1-3, and the adapter gradients of section 3.2).

The frozen weight arrives already split offline (Eq. 1): the residual R and
the stabilizer factors L1, L2.  Q(R) is computed once at construction.  The
trainable LoRA factors A and B are the module's only parameters; R, L1 and L2
get no gradients (section 3.1: the backbone and stabilizer branches are
frozen, differentiable pathways).

Every step runs in libft through the binding in ``ops``:

  forward:   Q(X) and T = X [L1 | A] in one pass, then
             Y = deq(Q(X)) deq(Q(R))^T + T [L2; B]                    (Eq. 2)
  backward:  Q(G) and V = G [L2; B]^T in one pass, then
             dX = deq(Q(G)) deq(Q(R)) + V [L1 | A]^T                  (Eq. 3)
             dA = X^T V_A,  dB = (X A)^T G                            (section 3.2)

Factors are stored rank-major as the C ABI takes them: L1t = L1^T [rs, K],
At = A^T [r, K], L2 [rs, N], B [r, N], all bf16.  X, Y and the incoming
gradient are bf16 [M, K] / [M, N] (M, K, N multiples of 16).  The kernels
produce fp32 adapter gradients; autograd delivers them in the parameters'
dtype (bf16), and the fp32 values of the last backward stay readable as
``last_grad_At`` / ``last_grad_B``.
"""
from __future__ import annotations

import torch

from . import ops


class _TripleBranch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, At, B, layer):
        if X.dtype != torch.bfloat16 or X.dim() != 2:
            raise ValueError("X must be a 2-D bf16 tensor [tokens, in_features]")
        X = X.contiguous()
        M = X.shape[0]
        T, xq, xs = ops.quant_lowrank(X, layer.L1t, At)
        Y = ops.linear_fwd(xq, xs, layer.rq, layer.rs_, T, layer.L2, B, M, layer.N, layer.K,
                           out_dtype=torch.bfloat16)
        ctx.layer = layer
        ctx.save_for_backward(X, T, At, B)
        return Y

    @staticmethod
    def backward(ctx, gY):
        X, T, At, B = ctx.saved_tensors
        layer = ctx.layer
        if gY.dtype != torch.bfloat16:
            raise ValueError(f"the gradient of Y must be bf16, got {gY.dtype}")
        G = gY.contiguous()
        M = X.shape[0]
        V, gq, gs = ops.quant_lowrank(G, layer.L2, B)
        dX, dAt, dB = ops.linear_bwd(gq, gs, layer.rqc, layer.rsct, V, layer.L1t, At, X, G, T, M, layer.N,
                                     layer.K, out_dtype=torch.bfloat16)
        layer.last_grad_At, layer.last_grad_B = dAt, dB
        return dX, dAt, dB, None


class Linear(torch.nn.Module):
    """W4A4G4 triple-branch linear: Y = Q(X) Q(R)^T + X L1 L2 + X A B.

    R      bf16 [N, K] (frozen residual, out x in)
    L1t    bf16 [rs, K], L2 bf16 [rs, N] (frozen stabilizer, rank-major)
    At     bf16 [r, K], B bf16 [r, N]    (trainable LoRA factors, rank-major)
    """

    def __init__(self, R: torch.Tensor, L1t: torch.Tensor, L2: torch.Tensor, At: torch.Tensor, B: torch.Tensor):
        super().__init__()
        self.N, self.K = R.shape
        # offline: Q(R) with both code layouts and the transposed scale grid
        rq, rqc, rs_, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
        for name, t in (("rq", rq), ("rqc", rqc), ("rs_", rs_), ("rsct", rsct), ("L1t", L1t), ("L2", L2)):
            self.register_buffer(name, t)
        self.At = torch.nn.Parameter(At)
        self.B = torch.nn.Parameter(B)
        self.last_grad_At = None
        self.last_grad_B = None

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return _TripleBranch.apply(X, self.At, self.B, self)
