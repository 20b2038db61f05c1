"""Chained stacks on the GPU against the oracle's own chain, at full size.

* MLP pair (Student-t activations): up 3072 -> 12288, GELU, down 12288 -> 3072,
  M = 4608 tokens.
* Double-stream block stack: image (M = 4096) and text (M = 512) streams, each
  with qkv 3072 -> 9216 and proj 3072 -> 3072 on fresh seeded inputs and
  up -> GELU -> down chained (attention and modulation are not part of the path).

Where the GPU hands a bf16 tensor to the next layer (Y_up, h, dX_down, dY_up),
the oracle rounds its fp64 value to bf16 at the same point and continues from
that.  Final outputs are fp32 on the GPU and compared by relative Frobenius
error against fp64 (contract 2e-3); the bf16 intermediates are compared with
the oracle's bf16-rounded values.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
_CACHE = {}


def _config(cfg):
    if cfg not in _CACHE:
        _CACHE[cfg] = {d["spec"].name: d for d in synth.config_linears(cfg)}
    return _CACHE[cfg]


class GpuLayer:
    """Device-side prepared layer: Q(R) (codes in both layouts, and the
    pair-merged operands of R and R^T), rank-major factors.

    path "op": the GEMMs read the pair-merged operands; the quantizer and the
    down-projection run as separate passes.  path "fused": the default path of
    the library -- one pass over X (G) writes Q(X) (Q(G)) and T (V), and the
    GEMMs read E2M1 codes + block scales."""

    def __init__(self, d, path="op"):
        from bit_quantized_lora_amd import ops
        self.ops, self.path = ops, path
        self.N, self.K = d["R"].shape
        Rd = dev_bf16(d["R"])
        self.ro = ops.quant_block16_op(Rd, op_rm=True, op_cm=True)
        self.rq, self.rqc, self.rs, self.rsct = ops.quant_block16(Rd, rm=True, cm=True, scales_cm=True)
        self.L1t = dev_bf16(np.ascontiguousarray(d["L1"].T))
        self.At = dev_bf16(np.ascontiguousarray(d["A"].T))
        self.L2, self.B = dev_bf16(d["L2"]), dev_bf16(d["B"])

    def fwd(self, X, out_dtype):
        o = self.ops
        M = X.shape[0]
        if self.path == "fused":
            T, xq, xs = o.quant_lowrank(X, self.L1t, self.At)
            Y = o.linear_fwd(xq, xs, self.rq, self.rs, T, self.L2, self.B, M, self.N, self.K, out_dtype=out_dtype)
            return Y, T
        xo = o.quant_block16_op(X, op_rm=True)
        T = o.lowrank_fused(X, self.L1t, self.At)
        Y = o.linear_fwd_op(xo["op_rm"], xo["op_rm_scales"], self.ro["op_rm"], self.ro["op_rm_scales"], T, self.L2,
                            self.B, M, self.N, self.K, out_dtype=out_dtype)
        return Y, T

    def fwd_codes_gelu(self, X):
        """Forward on the E2M1-codes GEMM path with the MLP fusion epilogue:
        (Y bf16, h bf16, Q(h) codes, Q(h) scales, T)."""
        o = self.ops
        M = X.shape[0]
        xq, _, xs = o.quant_block16(X, rm=True, cm=False)
        T = o.lowrank_fused(X, self.L1t, self.At)
        Y, H, hc, hs = o.linear_fwd_gelu(xq, xs, self.rq, self.rs, T, self.L2, self.B, M, self.N, self.K)
        return Y, H, hc, hs, T

    def fwd_codes_given_q(self, X, xq, xs, out_dtype):
        """Forward on the codes path from a Q(X) computed elsewhere."""
        o = self.ops
        M = X.shape[0]
        T = o.lowrank_fused(X, self.L1t, self.At)
        return o.linear_fwd(xq, xs, self.rq, self.rs, T, self.L2, self.B, M, self.N, self.K,
                            out_dtype=out_dtype), T

    def bwd(self, G, X, T, out_dtype):
        o = self.ops
        M = G.shape[0]
        if self.path == "fused":
            V, gq, gs = o.quant_lowrank(G, self.L2, self.B)
            return o.linear_bwd(gq, gs, self.rqc, self.rsct, V, self.L1t, self.At, X, G, T, M, self.N, self.K,
                                out_dtype=out_dtype)
        go = o.quant_block16_op(G, op_rm=True)
        V = o.lowrank_fused(G, self.L2, self.B)
        dX, dAt, dB = o.linear_bwd_op(go["op_rm"], go["op_rm_scales"], self.ro["op_cm"], self.ro["op_cm_scales"], V,
                                      self.L1t, self.At, X, G, T, M, self.N, self.K, out_dtype=out_dtype)
        return dX, dAt, dB


class OracleLayer:
    def __init__(self, d):
        rc, rsc = O.quantize_block16(d["R"])
        self.Rhat = O.dequantize(rc, rsc, "pow2")
        self.f = {k: O.bf16_to_f64(d[k]) for k in ("L1", "L2", "A", "B")}

    def fwd(self, Xbits):
        xc, xs = O.quantize_block16(Xbits)
        f = self.f
        return O.linear_fwd(O.dequantize(xc, xs, "pow2"), self.Rhat, O.bf16_to_f64(Xbits),
                            f["L1"], f["L2"], f["A"], f["B"])

    def bwd(self, Gbits, Xbits):
        gc, gs = O.quantize_block16(Gbits)
        f = self.f
        g = O.linear_bwd(O.dequantize(gc, gs, "pow2"), self.Rhat, O.bf16_to_f64(Gbits),
                         O.bf16_to_f64(Xbits), f["L1"], f["L2"], f["A"], f["B"])
        g["dA"] = g["dA"].T  # compare in the rank-major layout of the ABI
        return g


def _check(label, got, ref, bf16=False):
    g = O.bf16_to_f64(host(got)) if bf16 else host(got).astype(np.float64)
    r = O.bf16_to_f64(ref) if bf16 else ref
    e = O.rel_frob(g, r)
    say(f"[chain] {label}: rel-Frobenius {e:.2e}")
    assert e <= TOL, f"{label}: error {e:.3e} above 2e-3"
    return e


def _single(label, d, path="op"):
    """A standalone linear of the stack (fresh seeded input): fwd + bwd."""
    import torch
    say(f"[chain] {label} M={d['X'].shape[0]} K={d['R'].shape[1]} N={d['R'].shape[0]} path={path}")
    L, Lo = GpuLayer(d, path), OracleLayer(d)
    X, G = dev_bf16(d["X"]), dev_bf16(d["G"])
    Y, T = L.fwd(X, torch.float32)
    dX, dAt, dB = L.bwd(G, X, T, torch.float32)
    _check(f"{label} Y", Y, Lo.fwd(d["X"]))
    ref = Lo.bwd(d["G"], d["X"])
    _check(f"{label} dX", dX, ref["dX"])
    _check(f"{label} dA", dAt, ref["dA"])
    _check(f"{label} dB", dB, ref["dB"])


def _mlp_chain(label, up, down, path="op"):
    """up -> GELU -> down forward, then backward from down's seeded gradient."""
    import torch
    from bit_quantized_lora_amd import ops
    M = up["X"].shape[0]
    say(f"[chain] {label} MLP chain M={M} path={path}")
    Lu, Ld = GpuLayer(up, path), GpuLayer(down, path)
    X, G2 = dev_bf16(up["X"]), dev_bf16(down["G"])
    Y1, T1 = Lu.fwd(X, torch.bfloat16)
    h = ops.gelu_fwd(Y1)
    Y2, T2 = Ld.fwd(h, torch.float32)
    dh, dA2, dB2 = Ld.bwd(G2, h, T2, torch.bfloat16)
    dY1 = ops.gelu_bwd(Y1, dh)
    dX1, dA1, dB1 = Lu.bwd(dY1, X, T1, torch.float32)
    torch.cuda.synchronize()

    Lou, Lod = OracleLayer(up), OracleLayer(down)
    y1 = O.f64_to_bf16_bits(Lou.fwd(up["X"]))
    hb = O.f64_to_bf16_bits(O.gelu(O.bf16_to_f64(y1)))
    y2 = Lod.fwd(hb)
    gd = Lod.bwd(down["G"], hb)
    dhb = O.f64_to_bf16_bits(gd["dX"])
    dy1 = O.f64_to_bf16_bits(O.gelu_grad(O.bf16_to_f64(y1)) * O.bf16_to_f64(dhb))
    gu = Lou.bwd(dy1, up["X"])

    _check(f"{label} Y_up (bf16)", Y1, y1, bf16=True)
    _check(f"{label} h = GELU(Y_up) (bf16)", h, hb, bf16=True)
    _check(f"{label} Y_down", Y2, y2)
    _check(f"{label} dX_down = dh (bf16)", dh, dhb, bf16=True)
    _check(f"{label} dA_down", dA2, gd["dA"])
    _check(f"{label} dB_down", dB2, gd["dB"])
    _check(f"{label} dY_up (bf16)", dY1, dy1, bf16=True)
    _check(f"{label} dX_up", dX1, gu["dX"])
    _check(f"{label} dA_up", dA1, gu["dA"])
    _check(f"{label} dB_up", dB1, gu["dB"])


@pytest.mark.parametrize("path", ["fused", "op"])
def test_mlp_pair_chain_full_size(path):
    require_gpu()
    c = _config("c3")
    _mlp_chain("mlp-pair", c["c3-up"], c["c3-down"], path)


@pytest.mark.parametrize("path", ["fused", "op"])
@pytest.mark.parametrize("stream", ["txt", "img"])
def test_block_stack_full_size(stream, path):
    """All four linears of a stream (qkv, proj, then up -> GELU -> down chained),
    on the library's default one-pass codes path and on the pair-merged
    operand path."""
    require_gpu()
    c = _config("c5")
    _single(f"c5-{stream}-qkv", c[f"c5-{stream}-qkv"], path)
    _single(f"c5-{stream}-proj", c[f"c5-{stream}-proj"], path)
    _mlp_chain(f"c5-{stream}", c[f"c5-{stream}-up"], c[f"c5-{stream}-down"], path)


def _fused_fc1_matches_separate(M, K, N, rs, r, seed):
    """ft_linear_fwd_gelu against ft_linear_fwd -> ft_gelu_fwd -> ft_quant_block16.

    The epilogue's own results bit for bit: h = GELU(Y) of its Y (ft_gelu_fwd on
    the fused Y) and Q(h) (ft_quant_block16 of the fused h).  Y against the
    separate GEMM: within one bf16 step per element (the two launches may add
    the low-rank term at different points of the sum; plus fp32 summation noise
    near zero), and identical where both launches take the pipelined kernel
    (it adds the low-rank term first whatever the tile or epilogue)."""
    import torch
    from bit_quantized_lora_amd import ops
    rng = np.random.default_rng(seed)
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_dist="t3")
    d = synth.make_linear(spec, rng)
    say(f"[mlp-fusion] M={M} K={K} N={N} rs={rs} r={r}")
    L = GpuLayer(d)
    X = dev_bf16(d["X"])
    Yf, Hf, hcf, hsf, T = L.fwd_codes_gelu(X)
    xq, _, xs = ops.quant_block16(X, rm=True, cm=False)
    Ys, _ = L.fwd_codes_given_q(X, xq, xs, torch.bfloat16)
    Hg = ops.gelu_fwd(Yf)
    hcg, _, hsg = ops.quant_block16(Hf, rm=True, cm=False)
    torch.cuda.synchronize()
    for name, a, b in (("h", Hf, Hg), ("Q(h) codes", hcf, hcg), ("Q(h) scales", hsf, hsg)):
        ha, hb = host(a.view(torch.int16) if a.dtype == torch.bfloat16 else a), \
                 host(b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
        diff = int(np.count_nonzero(ha != hb))
        say(f"[mlp-fusion]   {name} (epilogue vs separate kernels on its Y): {diff} of {ha.size} differ")
        assert diff == 0, f"{name}: {diff} differing elements"
    yf, ys = O.bf16_to_f64(host(Yf)), O.bf16_to_f64(host(Ys))
    ndiff = int(np.count_nonzero(yf != ys))
    # one bf16 step of the element, plus fp32 summation-order noise in absolute
    # terms (an element that cancels to near zero keeps the rounding error of
    # its much larger terms)
    atol = 1e-5 * float(np.sqrt(np.mean(ys * ys)))
    worst = float(np.max(np.abs(yf - ys) - 2.0 ** -7 * np.maximum(np.abs(yf), np.abs(ys)) - atol))
    say(f"[mlp-fusion]   Y: {ndiff} of {yf.size} differ from the separate GEMM, worst excess over one step {worst:.2e}")
    assert worst <= 0.0, "Y differs from the separate GEMM by more than one bf16 step"
    if K % 128 == 0:   # the same pipelined kernel both ways: the same sum order
        assert ndiff == 0, "same kernel for both launches, yet Y differs"


@pytest.mark.parametrize("shape", [
    (4608, 3072, 12288, 32, 16),   # MLP up at full size: wide tiles
    (528, 1024, 784, 16, 16),      # 128 x 128 tiles, ragged N
    (4592, 384, 12272, 16, 16),    # wide tiles, ragged M and N, 3 stages
    (256, 272, 512, 16, 16),       # K % 128 != 0: the separate kernels
], ids=lambda s: "x".join(map(str, s[:3])))
def test_fused_fc1_epilogue_matches_separate_kernels(shape):
    require_gpu()
    M, K, N, rs, r = shape
    _fused_fc1_matches_separate(M, K, N, rs, r, seed=M + K + N)


def test_mlp_pair_chain_fused_fc1_full_size():
    """The MLP pair with the fused first linear (codes GEMM path): the down layer
    consumes Q(h) from the up layer's epilogue; every result against the oracle's
    chain."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    c = _config("c3")
    up, down = c["c3-up"], c["c3-down"]
    say("[chain] mlp-pair fused FC1 (codes path)")
    Lu, Ld = GpuLayer(up), GpuLayer(down)
    X, G2 = dev_bf16(up["X"]), dev_bf16(down["G"])
    Y1, h, hc, hs, T1 = Lu.fwd_codes_gelu(X)
    Y2, T2 = Ld.fwd_codes_given_q(h, hc, hs, torch.float32)
    dh, dA2, dB2 = Ld.bwd(G2, h, T2, torch.bfloat16)
    dY1 = ops.gelu_bwd(Y1, dh)
    dX1, dA1, dB1 = Lu.bwd(dY1, X, T1, torch.float32)
    torch.cuda.synchronize()

    Lou, Lod = OracleLayer(up), OracleLayer(down)
    y1 = O.f64_to_bf16_bits(Lou.fwd(up["X"]))
    hb = O.f64_to_bf16_bits(O.gelu(O.bf16_to_f64(y1)))
    y2 = Lod.fwd(hb)
    gd = Lod.bwd(down["G"], hb)
    dhb = O.f64_to_bf16_bits(gd["dX"])
    dy1 = O.f64_to_bf16_bits(O.gelu_grad(O.bf16_to_f64(y1)) * O.bf16_to_f64(dhb))
    gu = Lou.bwd(dy1, up["X"])

    _check("fused Y_up (bf16)", Y1, y1, bf16=True)
    _check("fused h = GELU(Y_up) (bf16)", h, hb, bf16=True)
    _check("fused Y_down", Y2, y2)
    _check("fused dX_down = dh (bf16)", dh, dhb, bf16=True)
    _check("fused dA_down", dA2, gd["dA"])
    _check("fused dB_down", dB2, gd["dB"])
    _check("fused dY_up (bf16)", dY1, dy1, bf16=True)
    _check("fused dX_up", dX1, gu["dX"])
    _check("fused dA_up", dA1, gu["dA"])
    _check("fused dB_up", dB1, gu["dB"])


@pytest.mark.parametrize("case", [
    (4608, 12288, 32, 16),     # the MLP intermediate at full size, down-layer ranks
    (48, 400, 16, 16),         # a ragged last chunk of the reduction
    (272, 1040, 64, 64),       # two rank tiles, several splits
    (16, 16, 0, 16),
    (256, 384, 0, 0),          # no projection: GELU and Q(h) only
    (400, 1296, 48, 32),       # 128-row blocks with whole-line loads, ragged rows and reduction
    (4096, 12288, 32, 32),     # the image-stream MLP intermediate of the FLUX block, rank 64
], ids=lambda c: "x".join(map(str, c)))
def test_gelu_quant_lowrank_matches_separate_kernels(case):
    """The MLP fusion in the second linear's input pass: h, Q(h) and the
    down-projection equal ft_gelu_fwd -> ft_quant_lowrank bit for bit."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, K, ra, rb = case
    rng = np.random.default_rng(M + K + ra)
    y = synth.f32_to_bf16_bits((rng.standard_t(3, (M, K)) * 2).astype(np.float32))
    wa = synth.f32_to_bf16_bits(synth.make_tensor(rng, (ra, K), "normal", 0.02))
    wb = synth.f32_to_bf16_bits(synth.make_tensor(rng, (rb, K), "normal", 0.01))
    Y, Wa, Wb = dev_bf16(y), dev_bf16(wa), dev_bf16(wb)
    say(f"[mlp-fusion pass] M={M} K={K} ra={ra} rb={rb}")
    h, T, hc, hs = ops.gelu_quant_lowrank(Y, Wa, Wb)
    Hs = ops.gelu_fwd(Y)
    Ts, hcs, hss = ops.quant_lowrank(Hs, Wa, Wb)
    torch.cuda.synchronize()
    pairs = [("h", h.view(torch.int16), Hs.view(torch.int16)), ("codes", hc, hcs), ("scales", hs, hss)]
    if ra + rb:
        pairs.append(("T", T.view(torch.int32), Ts.view(torch.int32)))
    for name, a, b in pairs:
        diff = int(np.count_nonzero(host(a) != host(b)))
        assert diff == 0, f"{name}: {diff} differing elements"


def test_mlp_pair_chain_fused_pass_full_size():
    """The MLP pair with GELU, Q(h) and the down layer's T from one pass over
    Y_up (ft_gelu_quant_lowrank); every result against the oracle's chain."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    c = _config("c3")
    up, down = c["c3-up"], c["c3-down"]
    say("[chain] mlp-pair fused GELU + quantize + project pass")
    Lu, Ld = GpuLayer(up), GpuLayer(down)
    X, G2 = dev_bf16(up["X"]), dev_bf16(down["G"])
    xq, _, xs = ops.quant_block16(X, rm=True, cm=False)
    Y1, T1 = Lu.fwd_codes_given_q(X, xq, xs, torch.bfloat16)
    h, T2, hc, hs = ops.gelu_quant_lowrank(Y1, Ld.L1t, Ld.At)
    M = h.shape[0]
    Y2 = ops.linear_fwd(hc, hs, Ld.rq, Ld.rs, T2, Ld.L2, Ld.B, M, Ld.N, Ld.K)
    dh, dA2, dB2 = Ld.bwd(G2, h, T2, torch.bfloat16)
    dY1 = ops.gelu_bwd(Y1, dh)
    dX1, dA1, dB1 = Lu.bwd(dY1, X, T1, torch.float32)
    torch.cuda.synchronize()

    Lou, Lod = OracleLayer(up), OracleLayer(down)
    y1 = O.f64_to_bf16_bits(Lou.fwd(up["X"]))
    hb = O.f64_to_bf16_bits(O.gelu(O.bf16_to_f64(y1)))
    y2 = Lod.fwd(hb)
    gd = Lod.bwd(down["G"], hb)
    dhb = O.f64_to_bf16_bits(gd["dX"])
    dy1 = O.f64_to_bf16_bits(O.gelu_grad(O.bf16_to_f64(y1)) * O.bf16_to_f64(dhb))
    gu = Lou.bwd(dy1, up["X"])

    _check("pass Y_up (bf16)", Y1, y1, bf16=True)
    _check("pass h = GELU(Y_up) (bf16)", h, hb, bf16=True)
    _check("pass Y_down", Y2, y2)
    _check("pass dX_down = dh (bf16)", dh, dhb, bf16=True)
    _check("pass dA_down", dA2, gd["dA"])
    _check("pass dB_down", dB2, gd["dB"])
    _check("pass dY_up (bf16)", dY1, dy1, bf16=True)
    _check("pass dX_up", dX1, gu["dX"])
    _check("pass dA_up", dA1, gu["dA"])
    _check("pass dB_up", dB1, gu["dB"])
