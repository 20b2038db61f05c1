"""The autograd module (bit_quantized_lora_amd.linear.Linear) against the oracle:
Y from forward, dX and the LoRA gradients from backward; R, L1, L2 get none."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.mark.parametrize("case", ["c1", "ragged"])
def test_linear_module_forward_backward(case):
    require_gpu()
    import torch
    from bit_quantized_lora_amd.linear import Linear
    if case == "c1":
        d = synth.config_linears("c1")[0]
    else:
        spec = synth.LinearSpec("t", 272, 384, 528, 32, 16, x_dist="t3")
        d = synth.make_linear(spec, np.random.default_rng(272))
    M, K = d["X"].shape
    N = d["R"].shape[0]
    say(f"[autograd] {case} M={M} K={K} N={N}")
    layer = Linear(dev_bf16(d["R"]), dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(d["L2"]),
                   dev_bf16(np.ascontiguousarray(d["A"].T)), dev_bf16(d["B"]))
    assert [n for n, p in layer.named_parameters()] == ["At", "B"]
    X = dev_bf16(d["X"]).requires_grad_(True)
    Y = layer(X)
    Y.backward(dev_bf16(d["G"]))
    torch.cuda.synchronize()

    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "R", "L1", "L2", "A", "B", "G")}
    rc, rsc = O.quantize_block16(d["R"]); xc, xs = O.quantize_block16(d["X"]); gc, gs = O.quantize_block16(d["G"])
    Rhat, Xhat, Ghat = (O.dequantize(c, s, "pow2") for c, s in ((rc, rsc), (xc, xs), (gc, gs)))
    Yo = O.linear_fwd(Xhat, Rhat, f["X"], f["L1"], f["L2"], f["A"], f["B"])
    go = O.linear_bwd(Ghat, Rhat, f["G"], f["X"], f["L1"], f["L2"], f["A"], f["B"])
    checks = {
        "Y": (O.bf16_to_f64(host(Y.detach())), Yo),
        "dX": (O.bf16_to_f64(host(X.grad)), go["dX"]),
        "dA (bf16 grad)": (O.bf16_to_f64(host(layer.At.grad)), go["dA"].T),
        "dB (bf16 grad)": (O.bf16_to_f64(host(layer.B.grad)), go["dB"]),
        "dA (fp32)": (host(layer.last_grad_At).astype(np.float64), go["dA"].T),
        "dB (fp32)": (host(layer.last_grad_B).astype(np.float64), go["dB"]),
    }
    for k, (got, ref) in checks.items():
        e = O.rel_frob(got, ref)
        say(f"[autograd] {case} {k}: rel-Frobenius {e:.2e}")
        assert e <= TOL, f"{k}: {e:.3e}"
        if "fp32" in k:
            assert e <= 1e-4
    # frozen buffers carry no gradient
    assert all(not b.requires_grad for b in layer.buffers())
