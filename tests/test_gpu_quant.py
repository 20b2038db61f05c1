"""Bit-exact parity of ft_quant_block16 (HIP) against the CPU oracle."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _check(bits, mode, label):
    from bit_quantized_lora_amd import ops
    say(f"[quant] {label} {bits.shape} mode={mode}")
    x = dev_bf16(bits)
    rm, cm, sc, sct = ops.quant_block16(x, mode=mode, rm=True, cm=True, scales_cm=True)
    codes, scales = O.quantize_block16(bits, mode)
    got_rm, got_cm, got_sc = host(rm), host(cm), host(sc)
    # the transposed scale grid is the same grid, transposed (Q(x^T) = Q(x)^T)
    assert np.array_equal(host(sct), got_sc.T), f"{label}: transposed scale grid differs"
    assert np.array_equal(got_rm, O.pack_rm(codes)), f"{label}: row-major codes differ"
    assert np.array_equal(got_cm, O.pack_cm(codes)), f"{label}: column-major codes differ"
    if mode == "pow2":
        assert np.array_equal(got_sc, scales), f"{label}: scales differ"
    else:
        assert np.array_equal(got_sc.view(np.uint32), np.asarray(scales).view(np.uint32)), f"{label}: scales differ"
    # single-layout variants write the same bytes
    rm2, _, sc2 = ops.quant_block16(x, mode=mode, rm=True, cm=False)
    _, cm3, sc3 = ops.quant_block16(x, mode=mode, rm=False, cm=True)
    assert np.array_equal(host(rm2), got_rm) and np.array_equal(host(cm3), got_cm)
    assert np.array_equal(host(sc2), got_sc) and np.array_equal(host(sc3), got_sc)


@pytest.mark.parametrize("mode", ["pow2", "f32"])
@pytest.mark.parametrize("kind", ["zeros", "negzeros", "subnormal", "ties", "huge", "mixed"])
def test_quant_edge_tensors(kind, mode):
    require_gpu()
    _check(synth.edge_tensor(kind, 160, 272), mode, f"edge:{kind}")


@pytest.mark.parametrize("mode", ["pow2", "f32"])
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (144, 400), (256, 128), (400, 144)])
def test_quant_ragged_shapes(shape, mode):
    require_gpu()
    rng = np.random.default_rng(shape[0] * 1000 + shape[1])
    x = synth.make_tensor(rng, shape, "t3")
    _check(synth.f32_to_bf16_bits(x), mode, f"ragged{shape}")


@pytest.mark.parametrize("mode", ["pow2", "f32"])
def test_quant_config1_tensors(mode):
    require_gpu()
    d = synth.config_linears("c1")[0]
    for name in ("X", "R", "G"):
        _check(d[name], mode, f"c1:{name}")


def test_quant_full_size_config_tensors_sampled():
    """Full-size X, G and R of the MLP-up and QKV configs, quantized in one launch;
    a sample of 16-row strips is re-derived by the oracle (Q is block-local)."""
    require_gpu()
    from bit_quantized_lora_amd import ops
    for cfg in ("c3", "c4"):
        d = synth.config_linears(cfg)[0]
        for name in ("X", "G", "R"):
            bits = d[name]
            rows, cols = bits.shape
            say(f"[quant] full {cfg}:{name} {bits.shape}")
            rm, cm, sc = ops.quant_block16(dev_bf16(bits), mode="pow2", rm=True, cm=True)
            got_rm, got_cm, got_sc = host(rm), host(cm), host(sc)
            rng = np.random.default_rng(rows + cols)
            strips = np.unique(np.concatenate([[0, rows // 16 - 1], rng.integers(0, rows // 16, 6)]))
            for s in strips:
                sl = slice(16 * s, 16 * s + 16)
                codes, scales = O.quantize_block16(bits[sl], "pow2")
                assert np.array_equal(got_rm[sl], O.pack_rm(codes))
                assert np.array_equal(got_sc[s], scales[0])
                assert np.array_equal(got_cm[:, 8 * s:8 * s + 8], O.pack_cm(codes))


# --------------------------------------------------------------------------
# pair-merged GEMM operands (bit-exact against the oracle's encoding)
# --------------------------------------------------------------------------
def _check_op(bits, label):
    from bit_quantized_lora_amd import ops
    say(f"[quant-op] {label} {bits.shape}")
    x = dev_bf16(bits)
    got = ops.quant_block16_op(x, codes_rm=True, codes_cm=True, op_rm=True, op_cm=True)
    codes, scales = O.quantize_block16(bits, "pow2")
    assert np.array_equal(host(got["codes_rm"]), O.pack_rm(codes)), f"{label}: codes_rm"
    assert np.array_equal(host(got["codes_cm"]), O.pack_cm(codes)), f"{label}: codes_cm"
    assert np.array_equal(host(got["scales"]), scales), f"{label}: scales"
    op, osc = O.operand_merge(codes, scales)
    assert np.array_equal(host(got["op_rm_scales"]), osc), f"{label}: op_rm scales"
    assert np.array_equal(host(got["op_rm"]), op), f"{label}: op_rm bytes"
    opt, osct = O.operand_merge(codes.T, scales.T)
    assert np.array_equal(host(got["op_cm_scales"]), osct), f"{label}: op_cm scales"
    assert np.array_equal(host(got["op_cm"]), opt), f"{label}: op_cm bytes"
    # operand-only launches write the same bytes
    only = ops.quant_block16_op(x, op_rm=True, op_cm=False)
    assert np.array_equal(host(only["op_rm"]), op) and np.array_equal(host(only["op_rm_scales"]), osc)
    only = ops.quant_block16_op(x, op_rm=False, op_cm=True)
    assert np.array_equal(host(only["op_cm"]), opt) and np.array_equal(host(only["op_cm_scales"]), osct)


@pytest.mark.parametrize("kind", ["zeros", "negzeros", "subnormal", "ties", "huge", "mixed"])
def test_operand_edge_tensors(kind):
    require_gpu()
    _check_op(synth.edge_tensor(kind, 160, 272), f"edge:{kind}")


@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (144, 400), (256, 128), (400, 144), (128, 528)])
def test_operand_ragged_shapes(shape):
    require_gpu()
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    _check_op(synth.f32_to_bf16_bits(synth.make_tensor(rng, shape, "t3")), f"ragged{shape}")


def test_operand_outlier_channels_unmerged_pairs():
    """Activation outlier channels (x50, x100) open exponent gaps past the merge
    range: a mix of merged and unmerged pairs."""
    require_gpu()
    for cfg in ("c2", "c4"):
        d = synth.config_linears(cfg, scale_m=256)[0]
        codes, scales = O.quantize_block16(d["X"], "pow2")
        _, osc = O.operand_merge(codes, scales)
        assert np.any(osc[:, 0::2] != osc[:, 1::2]), "expected some unmerged pairs"
        _check_op(d["X"], f"{cfg}:X")


def test_operand_full_size_sampled():
    """Full-size R of the MLP-up linear and G of the QKV config, one launch each;
    sampled 16-row strips (operand of x) and 16-column strips (operand of x^T)."""
    require_gpu()
    from bit_quantized_lora_amd import ops
    for cfg, name in (("c3", "R"), ("c4", "G")):
        bits = synth.config_linears(cfg)[0][name]
        rows, cols = bits.shape
        say(f"[quant-op] full {cfg}:{name} {bits.shape}")
        got = ops.quant_block16_op(dev_bf16(bits), op_rm=True, op_cm=True)
        op_rm, sc_rm, op_cm, sc_cm = (host(got[k]) for k in ("op_rm", "op_rm_scales", "op_cm", "op_cm_scales"))
        rng = np.random.default_rng(rows + cols)
        for s in np.unique(np.concatenate([[0, rows // 16 - 1], rng.integers(0, rows // 16, 4)])):
            c, sc = O.quantize_block16(bits[16 * s:16 * s + 16])
            op, osc = O.operand_merge(c, sc)
            assert np.array_equal(op_rm[16 * s:16 * s + 16], op) and np.array_equal(sc_rm[s], osc[0])
        for s in np.unique(np.concatenate([[0, cols // 16 - 1], rng.integers(0, cols // 16, 4)])):
            c, sc = O.quantize_block16(bits[:, 16 * s:16 * s + 16])
            op, osc = O.operand_merge(c.T, sc.T)
            assert np.array_equal(op_cm[16 * s:16 * s + 16], op) and np.array_equal(sc_cm[s], osc[0])


def test_stream_reference_kernel():
    """ft_stream_2to1 (the quantizer's same-run streaming reference) writes the high
    byte of every 16-bit input."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    rng = np.random.default_rng(5)
    for n in (16, 4096 + 16, 3 * 1024 * 1024):
        x = rng.integers(0, 1 << 16, n, dtype=np.uint16)
        xt = torch.from_numpy(x.view(np.int16)).cuda()
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
        ops.stream_2to1(xt, out)
        assert np.array_equal(host(out), (x >> 8).astype(np.uint8))
