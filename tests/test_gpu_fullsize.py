"""Whole-tensor parity at the configs' full sizes.

* Q(.) of every config tensor (X, G and the residual R of each linear of
  configs 2-5), both code layouts and both scale grids, compared in full with
  the oracle's quantizer, row strip by row strip on the host; and the codes
  and scales the one-pass quantize + down-projection writes for X and G.
* Y and dX of the MLP-up linear (4608 x 3072 -> 12288) on the default codes
  path, compared in full.
* The benchmark's own step (the same Linear object bench.py times: one pass
  over X and G for Q and the down-projection, bf16 Y and dX, fp32 dA and dB)
  against the oracle, in full.

Codes and scales must be bit-exact.  fp32 outputs are held to the 2e-3
relative Frobenius contract and the 1e-4 precision budget; bf16 outputs to the
contract and, element by element, to one bf16 step of the oracle's value.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
BUDGET = 1e-4
STRIP = 2048          # host comparison chunk (rows)


def _config_tensors(cfg):
    """(name, bf16 bits) of every tensor the config quantizes: X of each linear
    (a seeded stand-in for the chained second linear of a pair), G, and R."""
    out = []
    for d in synth.config_linears(cfg):
        spec = d["spec"]
        if "X" not in d:
            d["X"] = synth.f32_to_bf16_bits(synth.make_tensor(np.random.default_rng(99), (spec.M, spec.K), "t3"))
        out.append((d, spec))
    return out


def _compare_quant_whole(bits, codes_rm, codes_cm, scales, scales_cm, label):
    """Every code and scale of Q(bits) against the oracle, STRIP rows at a time."""
    rows, cols = bits.shape
    crm, ccm, sc, sct = host(codes_rm), host(codes_cm) if codes_cm is not None else None, host(scales), \
        host(scales_cm) if scales_cm is not None else None
    for r0 in range(0, rows, STRIP):
        r1 = min(rows, r0 + STRIP)
        c, s = O.quantize_block16(bits[r0:r1], "pow2")
        assert np.array_equal(crm[r0:r1], O.pack_rm(c)), f"{label}: row-major codes differ in rows {r0}..{r1}"
        assert np.array_equal(sc[r0 // 16:r1 // 16], s), f"{label}: scales differ in rows {r0}..{r1}"
        if ccm is not None:
            assert np.array_equal(ccm[:, r0 // 2:r1 // 2], O.pack_cm(c)), f"{label}: column-major codes differ"
        if sct is not None:
            assert np.array_equal(sct[:, r0 // 16:r1 // 16], s.T), f"{label}: transposed scales differ"


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c5"])
def test_quantizer_whole_tensors_full_size(cfg):
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    for d, spec in _config_tensors(cfg):
        for name in ("X", "G", "R"):
            bits = d[name]
            say(f"[fullsize] Q({name}) of {spec.name} {bits.shape}")
            x = dev_bf16(bits)
            rm, cm, sc, sct = ops.quant_block16(x, rm=True, cm=True, scales_cm=True)
            _compare_quant_whole(bits, rm, cm, sc, sct, f"{spec.name} {name}")
            del rm, cm, sc, sct
            if name != "R":   # the one-pass quantize + down-projection of the step
                wa, wb = (d["L1"].T, d["A"].T) if name == "X" else (d["L2"], d["B"])
                _, codes, scales = ops.quant_lowrank(x, dev_bf16(np.ascontiguousarray(wa)),
                                                     dev_bf16(np.ascontiguousarray(wb)))
                torch.cuda.synchronize()
                _compare_quant_whole(bits, codes, None, scales, None, f"{spec.name} {name} (one pass)")
                del codes, scales
            del x
            torch.cuda.empty_cache()


def _oracle_full(d):
    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "R", "L1", "L2", "A", "B", "G")}
    rc, rsc = O.quantize_block16(d["R"])
    xc, xs = O.quantize_block16(d["X"])
    gc, gs = O.quantize_block16(d["G"])
    Rhat, Xhat, Ghat = O.dequantize(rc, rsc, "pow2"), O.dequantize(xc, xs, "pow2"), O.dequantize(gc, gs, "pow2")
    Y = O.linear_fwd(Xhat, Rhat, f["X"], f["L1"], f["L2"], f["A"], f["B"])
    g = O.linear_bwd(Ghat, Rhat, f["G"], f["X"], f["L1"], f["L2"], f["A"], f["B"])
    return {"Y": Y, "dX": g["dX"], "dA": g["dA"].T, "dB": g["dB"]}


def _check_f32(label, got, ref):
    e = O.rel_frob(got, ref)
    say(f"[fullsize] {label}: rel-Frobenius {e:.2e}")
    assert e <= TOL and e <= BUDGET, f"{label}: error {e:.3e}"


def _check_bf16(label, got_bits, ref):
    got = O.bf16_to_f64(got_bits)
    e = O.rel_frob(got, ref)
    # each element within one bf16 step of the exact value, plus the fp32
    # precision budget in absolute terms (elements that cancel to near zero
    # carry the fp32 accumulation error of their much larger terms)
    step = np.abs(ref) * 2.0 ** -7
    atol = BUDGET * float(np.sqrt(np.mean(ref * ref)))
    worst = float(np.max(np.abs(got - ref) - step - atol))
    say(f"[fullsize] {label} (bf16): rel-Frobenius {e:.2e}, worst excess over one step {worst:.2e}")
    assert e <= TOL, f"{label}: error {e:.3e} above 2e-3"
    assert worst <= 0.0, f"{label}: an element is more than one bf16 step from the oracle"


def test_mlp_up_codes_path_whole_outputs():
    """The MLP-up linear on the codes path (separate quantizer and down-projection
    passes, fp32 outputs): every element of Y and dX against the oracle."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    d = synth.config_linears("c3")[0]
    spec = d["spec"]
    M, K, N = spec.M, spec.K, spec.N
    say(f"[fullsize] {spec.name} codes path, whole Y and dX")
    X, R, G = dev_bf16(d["X"]), dev_bf16(d["R"]), dev_bf16(d["G"])
    L1t, At = dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(np.ascontiguousarray(d["A"].T))
    L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
    rq, rqc, rsc, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
    xq, _, xs = ops.quant_block16(X)
    T = ops.lowrank_fused(X, L1t, At)
    Y = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K)
    gq, _, gs = ops.quant_block16(G)
    V = ops.lowrank_fused(G, L2, B)
    dX, dAt, dB = ops.linear_bwd(gq, gs, rqc, rsct, V, L1t, At, X, G, T, M, N, K)
    torch.cuda.synchronize()
    ref = _oracle_full(d)
    _check_f32("Y", host(Y).astype(np.float64), ref["Y"])
    _check_f32("dX", host(dX).astype(np.float64), ref["dX"])
    _check_f32("dA", host(dAt).astype(np.float64), ref["dA"])
    _check_f32("dB", host(dB).astype(np.float64), ref["dB"])


def test_bench_step_against_oracle():
    """bench.py's Linear step (default path) on its first input set, against the
    oracle: bf16 Y and dX, fp32 dA and dB, every element."""
    require_gpu()
    import torch
    import bench
    spec, d = bench.make_inputs()
    say(f"[fullsize] bench step {spec.M}x{spec.K}x{spec.N} rs={spec.rs} r={spec.r}")
    lin = bench.Linear(spec, d, "fused")
    lin.forward()
    lin.backward()
    torch.cuda.synchronize()
    ref = _oracle_full(d)
    _check_bf16("Y", host(lin.Y), ref["Y"])
    _check_bf16("dX", host(lin.dX), ref["dX"])
    _check_f32("dA", host(lin.dAt).astype(np.float64), ref["dA"])
    _check_f32("dB", host(lin.dB).astype(np.float64), ref["dB"])
