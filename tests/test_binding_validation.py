"""The torch binding checks every tensor before its pointer reaches libft: a wrong
dtype, shape, layout or an undersized buffer raises ValueError instead of
becoming an out-of-bounds device access.  These run on the CPU: the checks
that can fail here come before the device check, and a well-formed CPU
tensor is rejected for not being on the device."""
import pytest
import torch

from bit_quantized_lora_amd import ops

bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
M, N, K, RS, R = 32, 48, 64, 16, 16


def z(shape, dt):
    return torch.zeros(shape, dtype=dt)


def fwd_args():
    return dict(xq_codes=z((M, K // 2), u8), xq_scales=z((M // 16, K // 16), u8),
                rq_codes=z((N, K // 2), u8), rq_scales=z((N // 16, K // 16), u8),
                T=z((M, RS + R), f32), L2=z((RS, N), bf), B=z((R, N), bf))


def bwd_args():
    return dict(gq_codes=z((M, N // 2), u8), gq_scales=z((M // 16, N // 16), u8),
                rq_codes_cm=z((K, N // 2), u8), rq_scales_cm=z((K // 16, N // 16), u8),
                V=z((M, RS + R), f32), L1t=z((RS, K), bf), At=z((R, K), bf),
                X=z((M, K), bf), G=z((M, N), bf), T=z((M, RS + R), f32))


def call_fwd(**over):
    a = fwd_args(); a.update(over)
    return ops.linear_fwd(a["xq_codes"], a["xq_scales"], a["rq_codes"], a["rq_scales"], a["T"], a["L2"],
                          a["B"], M, N, K, out=a.get("out", z((M, N), f32)))


def call_bwd(**over):
    a = bwd_args(); a.update(over)
    return ops.linear_bwd(a["gq_codes"], a["gq_scales"], a["rq_codes_cm"], a["rq_scales_cm"], a["V"], a["L1t"],
                          a["At"], a["X"], a["G"], a["T"], M, N, K, workspace=a.get("workspace"),
                          dX=a.get("dX", z((M, K), f32)), dAt=a.get("dAt", z((R, K), f32)),
                          dB=a.get("dB", z((R, N), f32)))


def test_wellformed_cpu_tensors_are_rejected_for_the_device():
    with pytest.raises(ValueError, match="device tensor"):
        call_fwd()
    with pytest.raises(ValueError, match="device tensor"):
        call_bwd(workspace=z((ops.linear_bwd_workspace(M, N, K, R) + 16,), u8))


@pytest.mark.parametrize("name,bad", [
    ("xq_codes", z((M, K // 2 - 16), u8)),          # undersized codes
    ("xq_codes", z((M, K // 2), torch.int8)),       # wrong dtype
    ("xq_scales", z((M // 16, K // 16), f32)),      # f32 scales with the pow2 rule
    ("rq_codes", z((N + 16, K // 2), u8)),          # wrong shape
    ("rq_scales", z((N // 16, K // 16 + 1), u8)),
    ("T", z((M, RS + R), bf)),                      # T must be fp32
    ("T", z((M, RS), f32)),
    ("L2", z((RS, N + 16), bf)),
    ("B", z((R + 1, N), bf)),                       # rank not a multiple of 16
    ("out", z((M, N - 16), f32)),                   # undersized output
    ("out", z((M, N), torch.float16)),              # unsupported output dtype
])
def test_forward_rejects_mismatched_tensors(name, bad):
    with pytest.raises(ValueError, match=name if name not in ("B",) else "B|ranks"):
        call_fwd(**{name: bad})


def test_forward_rejects_noncontiguous_views():
    codes = z((M, K), u8)[:, ::2]
    assert codes.shape == (M, K // 2) and not codes.is_contiguous()
    with pytest.raises(ValueError, match="xq_codes must be contiguous"):
        call_fwd(xq_codes=codes)
    out = z((N, M), f32).t()
    with pytest.raises(ValueError, match="out must be contiguous"):
        call_fwd(out=out)


@pytest.mark.parametrize("name,bad", [
    ("gq_codes", z((M, N // 2 - 8), u8)),
    ("gq_scales", z((M // 16 + 1, N // 16), u8)),
    ("rq_codes_cm", z((N, K // 2), u8)),            # row-major codes where column-major are expected
    ("rq_scales_cm", z((N // 16, K // 16), u8)),
    ("V", z((M, RS + R + 16), f32)),
    ("X", z((M, K), f32)),
    ("G", z((M, N - 16), bf)),
    ("dX", z((M, K - 16), f32)),
    ("dAt", z((R, K), bf)),                         # dAt must be fp32
    ("dB", z((R, N // 2), f32)),
    ("workspace", z((8,), u8)),                     # smaller than ft_linear_bwd_workspace
])
def test_backward_rejects_mismatched_tensors(name, bad):
    with pytest.raises(ValueError, match=name):
        call_bwd(**{name: bad})


def test_quantizer_rejects_bad_outputs():
    x = z((M, K), bf)
    with pytest.raises(ValueError, match="codes_rm"):
        ops.quant_block16(x, out=(z((M, K // 2 - 16), u8), None, z((M // 16, K // 16), u8)))
    with pytest.raises(ValueError, match="codes_cm"):
        ops.quant_block16(x, cm=True, out=(None, z((M, K // 2), u8), z((M // 16, K // 16), u8)))
    with pytest.raises(ValueError, match="scales"):
        ops.quant_block16(x, out=(z((M, K // 2), u8), None, z((M // 16, K // 16), f32)))
    with pytest.raises(ValueError, match="x must be"):
        ops.quant_block16(z((M, K), f32))
    with pytest.raises(ValueError, match="multiples of 16"):
        ops.quant_block16(z((M, K + 8), bf))
    with pytest.raises(ValueError, match="unit column stride"):
        ops.quant_block16(z((K, M), bf).t())


def test_lowrank_and_one_pass_reject_bad_buffers():
    x = z((M, K), bf)
    wa, wb = z((RS, K), bf), z((R, K), bf)
    with pytest.raises(ValueError, match="wa"):
        ops.lowrank_fused(x, z((RS, K + 16), bf), wb)
    with pytest.raises(ValueError, match="out"):
        ops.lowrank_fused(x, wa, wb, out=z((M, RS), f32))
    with pytest.raises(ValueError, match="codes"):
        ops.quant_lowrank(x, wa, wb, out=z((M, RS + R), f32), codes=z((M, K // 4), u8),
                          scales=z((M // 16, K // 16), u8))
    with pytest.raises(ValueError, match="scales"):
        ops.quant_lowrank(x, wa, wb, out=z((M, RS + R), f32), codes=z((M, K // 2), u8),
                          scales=z((M // 16, K // 8), u8))
    with pytest.raises(ValueError, match="ranks"):
        ops.lowrank_fused(x, z((80, K), bf), z((64, K), bf))


def test_group_and_gelu_bindings_reject_bad_buffers():
    x = z((M, K), bf)
    with pytest.raises(ValueError, match="group"):
        ops.quant_group(x, 8)
    with pytest.raises(ValueError, match="scales"):
        ops.quant_group(x, 16, out=(z((M, K // 2), u8), z((M, K // 32), u8)))
    with pytest.raises(ValueError, match="codes_t"):
        ops.requant_group_t(z((M, K // 2), u8), z((M, K // 16), u8), M, K, 16,
                            out=(z((M, K // 2), u8), z((K, M // 16), u8)))
    with pytest.raises(ValueError, match="out"):
        ops.gelu_fwd(x, out=z((M, K - 8), bf))
    with pytest.raises(ValueError, match="dh"):
        ops.gelu_bwd(x, z((M, K), f32))


def test_empty_operands_may_come_in_any_empty_shape():
    """A zero-sized dimension makes an operand empty; its tensor's shape is then free
    (the library takes NULL for it), so the checks pass and only the device check
    remains on the CPU."""
    e8 = z((0,), u8)
    with pytest.raises(ValueError, match="device tensor"):
        ops.linear_fwd(e8, e8, e8, e8, z((M, RS + R), f32), z((RS, N), bf), z((R, N), bf), M, N, 0,
                       out=z((M, N), f32))
