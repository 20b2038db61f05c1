"""The adapter gradients of FourTune section 3.2 (dA = X^T (G B^T), dB =
(X A)^T G) as ft_linear_bwd computes them: by extra workgroups of the dX GEMM
launch where the plan says so, else on the side stream.  Whole dA and dB
against fp64 products of the same bf16 inputs (the gradients' definitions),
dX against the oracle on sampled row strips, at sizes that take each branch of
the launch plan: workgroups beside a one-round GEMM, after a multi-round GEMM,
split token ranges, two 32-rank tiles with r not a multiple of 32, a ragged
last column strip, few tokens with the split dX GEMM, dB left out, and the
side-stream fallback."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

BUDGET = 1e-4   # fp32 accumulation of bf16 hi + lo products (16 significant bits of P)

# (M, K, N, rs, r), expected: "beside" (adapter workgroups start with the GEMM on
# the slots its last round leaves), "after" (up to one per slot, following a GEMM
# that leaves fewer than an eighth of the slots), "split" (token ranges), "side"
# (side stream)
CASES = [
    ((4608, 3072, 12288, 32, 16), "beside"),    # MLP up of a FLUX block (the benchmarked linear)
    ((4096, 4096, 1024, 16, 16), "after"),      # 242 wide dX tiles: 14 CUs left in the round
    ((16384, 1024, 1024, 32, 64), "split"),     # long token axis, 32 column strips
    ((4608, 3072, 3072, 16, 48), "beside"),     # two rank tiles, the second partly used
    ((400, 1040, 1152, 16, 16), "beside"),      # ragged: 16-column last strip, 400 tokens
    ((512, 3072, 9216, 32, 32), "beside"),      # 512 text tokens: 128 x 128 tiles, split dX GEMM
    ((512, 3072, 3072, 0, 64), "side"),         # r = 64 with 128 x 128 tiles: side stream
]


def _data(shape):
    M, K, N, rs, r = shape
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_dist="t3", x_outlier_count=4, x_outlier_mult=30.0)
    return synth.make_linear(spec, np.random.default_rng(M + 5 * K + 11 * N + r))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
def test_adapter_gradients_by_launch_plan(case):
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    shape, kind = case
    M, K, N, rs, r = shape
    plan = ops.linear_bwd_plan(M, N, K, r)
    say(f"[adapter] {shape} expect {kind}: plan {plan}")
    if kind == "side":
        assert plan[3] == 0
    else:
        assert plan[3] > 0
        if kind == "split":
            assert plan[4] > 1
        tiles = -(-M // plan[0]) * -(-K // plan[1]) * plan[2]
        slots = torch.cuda.get_device_properties(0).multi_processor_count * (2 if plan[0] == 128 else 1)
        free = -tiles % slots   # slots the GEMM's last round leaves
        if kind == "beside":
            assert free >= slots // 8 and plan[3] <= free
        elif kind == "after":
            assert free < slots // 8 and plan[3] == min(slots, (-(-K // 64) + -(-N // 64)) * plan[4])
    d = _data(shape)
    X, R, G = dev_bf16(d["X"]), dev_bf16(d["R"]), dev_bf16(d["G"])
    L1t, At = dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(np.ascontiguousarray(d["A"].T))
    L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
    _, rqc, _, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
    T, _, _ = ops.quant_lowrank(X, L1t, At)
    V, gq, gs = ops.quant_lowrank(G, L2, B)
    args = (gq, gs, rqc, rsct, V, L1t, At, X, G, T, M, N, K)
    dX, dAt, dB = ops.linear_bwd(*args)
    dX2, dAt2, dB2 = ops.linear_bwd(*args)
    _, dAt3, none = ops.linear_bwd(*args, skip_dB=True)
    torch.cuda.synchronize()
    assert none is None
    for a, b, name in ((dX, dX2, "dX"), (dAt, dAt2, "dA"), (dB, dB2, "dB")):
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), f"{name} not deterministic"
    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "G", "A", "B")}
    dA_ref = (f["X"].T @ (f["G"] @ f["B"].T)).T
    dB_ref = (f["X"] @ f["A"]).T @ f["G"]
    ea = O.rel_frob(host(dAt).astype(np.float64), dA_ref)
    eb = O.rel_frob(host(dB).astype(np.float64), dB_ref)
    ea3 = O.rel_frob(host(dAt3).astype(np.float64), dA_ref)
    # dX on 16-row strips against the oracle's Eq. 3
    rng = np.random.default_rng(M)
    strips = np.sort(rng.choice(M // 16, size=min(4, M // 16), replace=False))
    rows = (strips[:, None] * 16 + np.arange(16)[None, :]).ravel()
    rc, rsc = O.quantize_block16(d["R"])
    gc, gsc = O.quantize_block16(d["G"][rows])
    fl = {k: O.bf16_to_f64(d[k]) for k in ("L1", "L2")}
    ref_dx = O.linear_bwd(O.dequantize(gc, gsc, "pow2"), O.dequantize(rc, rsc, "pow2"), f["G"][rows],
                          f["X"][rows], fl["L1"], fl["L2"], f["A"], f["B"])["dX"]
    ex = O.rel_frob(host(dX).astype(np.float64)[rows], ref_dx)
    say(f"[adapter] {shape}: rel-Frobenius dA {ea:.2e} dB {eb:.2e} dA(no dB) {ea3:.2e} dX {ex:.2e}")
    for e, name in ((ea, "dA"), (eb, "dB"), (ea3, "dA without dB"), (ex, "dX")):
        assert e <= BUDGET, f"{shape}: {name} error {e:.3e}"
