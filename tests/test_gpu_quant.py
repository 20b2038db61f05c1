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
