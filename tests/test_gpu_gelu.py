"""GELU kernels (the activation between the MLP's linears) against the oracle's
fp64 GELU, over every bf16 value in [-12, 12] (exhaustive over that range:
normals of every exponent down to the smallest, both signs, and zero)."""
import numpy as np
import pytest

import oracle as O
from gpu_util import host, require_gpu, say

pytestmark = pytest.mark.gpu


def _all_bf16_in(lo, hi):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite patterns only
    v = O.bf16_to_f64(bits)
    keep = (v >= lo) & (v <= hi)
    b = bits[keep]
    pad = (-b.size) % 8
    return np.concatenate([b, np.zeros(pad, np.uint16)])


def _ulp_diff(a_bits, b_bits):
    """Distance in bf16 steps between two bf16 bit patterns (sign-magnitude order)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a_bits) - key(b_bits))


def test_gelu_fwd_bwd_against_oracle():
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    ybits = _all_bf16_in(-12.0, 12.0)
    y = torch.from_numpy(ybits.view(np.int16)).cuda().view(torch.bfloat16)
    ones = torch.ones_like(y)
    h = ops.gelu_fwd(y)
    dy = ops.gelu_bwd(y, ones)
    torch.cuda.synchronize()
    yv = O.bf16_to_f64(ybits)
    want_h = O.f64_to_bf16_bits(O.gelu(yv))
    want_d = O.f64_to_bf16_bits(O.gelu_grad(yv))
    got_h = host(h.view(torch.int16)).view(np.uint16)
    got_d = host(dy.view(torch.int16)).view(np.uint16)
    for name, got, want in (("GELU", got_h, want_h), ("GELU'", got_d, want_d)):
        d = _ulp_diff(got, want)
        exact = float(np.mean(d == 0))
        say(f"[gelu] {name}: {ybits.size} values, {100 * exact:.3f}% exact, max {int(d.max())} bf16 step(s) off")
        assert d.max() <= 1, f"{name}: {int(d.max())} bf16 steps off"
        assert exact >= 0.995, f"{name}: only {exact:.4f} of the values exact"
