"""Parity of the HIP triple-branch linear (forward, backward, low-rank, GELU)
against the fp64 CPU oracle.

Contract tolerance: relative Frobenius error <= 2e-3 for Y, dX, dA, dB (fp32
outputs).  A tighter precision budget (1e-4) is asserted as well: the 4-bit
products are exact and accumulate in fp32, and the low-rank intermediates are
carried as bf16 hi + lo pairs (16 significant bits), so anything above ~1e-5
indicates a lost term rather than rounding.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
BUDGET = 1e-4


def _gpu_linear(d, out_dtype=None, path="codes"):
    """Run quantize -> low-rank -> fwd and quantize -> low-rank -> bwd on the GPU.

    path "codes": the GEMMs read E2M1 codes + block scales (one 16-K block per
    32-K MFMA fragment); path "op": they read the pair-merged operands."""
    import torch
    from bit_quantized_lora_amd import ops
    out_dtype = out_dtype or torch.float32
    X, R, G = dev_bf16(d["X"]), dev_bf16(d["R"]), dev_bf16(d["G"])
    L1t = dev_bf16(np.ascontiguousarray(d["L1"].T))
    At = dev_bf16(np.ascontiguousarray(d["A"].T))
    L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
    M, K = d["X"].shape
    N = d["R"].shape[0]
    T = ops.lowrank_fused(X, L1t, At)
    V = ops.lowrank_fused(G, L2, B)
    if path == "codes":
        xq, _, xs = ops.quant_block16(X, rm=True, cm=False)
        rq, rqc, rsc, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
        Y = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K, out_dtype=out_dtype)
        gq, _, gs = ops.quant_block16(G, rm=True, cm=False)
        dX, dAt, dB = ops.linear_bwd(gq, gs, rqc, rsct, V, L1t, At, X, G, T, M, N, K, out_dtype=out_dtype)
    else:
        xo = ops.quant_block16_op(X, op_rm=True)
        ro = ops.quant_block16_op(R, op_rm=True, op_cm=True)
        Y = ops.linear_fwd_op(xo["op_rm"], xo["op_rm_scales"], ro["op_rm"], ro["op_rm_scales"], T, L2, B,
                              M, N, K, out_dtype=out_dtype)
        go = ops.quant_block16_op(G, op_rm=True)
        dX, dAt, dB = ops.linear_bwd_op(go["op_rm"], go["op_rm_scales"], ro["op_cm"], ro["op_cm_scales"], V, L1t,
                                        At, X, G, T, M, N, K, out_dtype=out_dtype)
    return {"Y": Y, "dX": dX, "dA": dAt, "dB": dB, "T": T, "V": V}


def _oracle_rows(d, rows):
    """Oracle Y and dX restricted to `rows` (a union of 16-row strips), full dA, dB."""
    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "R", "L1", "L2", "A", "B", "G")}
    rc, rsc = O.quantize_block16(d["R"])
    Rhat = O.dequantize(rc, rsc, "pow2")
    xc, xs = O.quantize_block16(d["X"][rows])
    gc, gs = O.quantize_block16(d["G"][rows])
    Xhat, Ghat = O.dequantize(xc, xs, "pow2"), O.dequantize(gc, gs, "pow2")
    Y = O.linear_fwd(Xhat, Rhat, f["X"][rows], f["L1"], f["L2"], f["A"], f["B"])
    g = O.linear_bwd(Ghat, Rhat, f["G"][rows], f["X"][rows], f["L1"], f["L2"], f["A"], f["B"])
    # adapter gradients need every token
    dB = (f["X"] @ f["A"]).T @ f["G"]
    dA = f["X"].T @ (f["G"] @ f["B"].T)
    return {"Y": Y, "dX": g["dX"], "dA": dA.T, "dB": dB}


def _compare(gpu, ref, rows, label):
    errs = {}
    for k in ("Y", "dX", "dA", "dB"):
        if ref[k].size == 0:
            continue
        got = host(gpu[k]).astype(np.float64)
        if k in ("Y", "dX"):
            got = got[rows]
        errs[k] = O.rel_frob(got, ref[k])
    say(f"[linear] {label} rel-Frobenius errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL, f"{label}: {k} error {e:.3e} above the 2e-3 contract"
        assert e <= BUDGET, f"{label}: {k} error {e:.3e} above the fp32 precision budget"
    return errs


SMALL = [
    # (M, K, N, rs, r): several 256-tiles, ragged tails, K % 32 == 16, rank edge cases
    (256, 256, 256, 16, 16),
    (144, 400, 272, 16, 16),
    (528, 176, 48, 32, 0),
    (48, 48, 48, 0, 16),
    (80, 528, 304, 64, 64),
    (16, 16, 16, 0, 0),
    (272, 1040, 528, 32, 32),
    # reduction lengths that are multiples of 128 (pipelined GEMM path, fwd and bwd),
    # with ragged M / N tiles and 1..9 pipeline stages
    (272, 384, 512, 16, 16),
    (48, 128, 128, 0, 16),
    (528, 256, 640, 32, 32),
    (304, 1152, 384, 16, 16),
]


@pytest.mark.parametrize("path", ["codes", "op"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_linear_small_and_ragged(shape, path):
    require_gpu()
    M, K, N, rs, r = shape
    rng = np.random.default_rng(M * 7 + K * 3 + N)
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_outlier_count=min(4, K), x_outlier_mult=30.0,
                            w_outlier_cols=min(2, K), w_outlier_mult=20.0)
    d = synth.make_linear(spec, rng)
    say(f"[linear] small {shape} path={path}")
    gpu = _gpu_linear(d, path=path)
    rows = np.arange(M)
    _compare(gpu, _oracle_rows(d, rows), rows, f"small{shape}/{path}")


def test_config1_full_and_bf16_and_determinism():
    require_gpu()
    import torch
    d = synth.config_linears("c1")[0]
    gpu = _gpu_linear(d)
    rows = np.arange(d["X"].shape[0])
    _compare(gpu, _oracle_rows(d, rows), rows, "c1")
    # run twice: identical bits
    again = _gpu_linear(d)
    for k in ("Y", "dX", "dA", "dB", "T", "V"):
        assert np.array_equal(host(gpu[k]).view(np.uint32), host(again[k]).view(np.uint32)), k
    # bf16 outputs are the round-to-nearest-even of the fp32 outputs
    gb = _gpu_linear(d, out_dtype=torch.bfloat16)
    for k in ("Y", "dX"):
        assert np.array_equal(host(gb[k]), synth.f32_to_bf16_bits(host(gpu[k]))), k


def test_lowrank_matches_oracle_products():
    require_gpu()
    from bit_quantized_lora_amd import ops
    for (M, K, ra, rb) in [(48, 400, 16, 16), (4608, 3072, 32, 16), (96, 12288, 64, 64), (32, 16, 0, 32)]:
        rng = np.random.default_rng(M + K)
        X = synth.f32_to_bf16_bits(synth.make_tensor(rng, (M, K), "t3"))
        Wa = synth.f32_to_bf16_bits(synth.make_tensor(rng, (ra, K), "normal", 0.05))
        Wb = synth.f32_to_bf16_bits(synth.make_tensor(rng, (rb, K), "normal", 0.01))
        say(f"[lowrank] {M}x{K} ra={ra} rb={rb}")
        out = host(ops.lowrank_fused(dev_bf16(X), dev_bf16(Wa), dev_bf16(Wb)))
        Xf = O.bf16_to_f64(X)
        ref = np.concatenate([Xf @ O.bf16_to_f64(Wa).T, Xf @ O.bf16_to_f64(Wb).T], axis=1)
        assert O.rel_frob(out, ref) < 1e-5


@pytest.mark.parametrize("case", [(144, 400, 16, 16), (272, 128, 32, 16), (16, 16, 0, 16), (528, 1040, 64, 64),
                                  (256, 384, 0, 0), (4608, 3072, 32, 16), (4608, 12288, 32, 16),
                                  (400, 1296, 48, 32), (208, 560, 32, 32), (160, 272, 64, 32), (144, 400, 64, 48),
                                  (4096, 3072, 32, 32)],
                         ids=lambda c: "x".join(map(str, c)))
def test_quant_lowrank_one_pass(case):
    """Q(in) and the down-projection from one read of the input: codes and scales
    bit-exact with the oracle's quantizer, the projection bit-identical to
    ft_lowrank_fused and within fp32 rounding of the oracle's product.  The ranks
    cover every launch layout: 64-row blocks with whole-line loads (rank <= 48),
    128-row blocks with whole-line loads (49..96, the boundary 96 included) and
    with fragment-layout loads (above 96), with row counts and reductions that
    end inside a block and inside a chunk."""
    require_gpu()
    from bit_quantized_lora_amd import ops
    M, K, ra, rb = case
    rng = np.random.default_rng(M * 3 + K)
    X = synth.f32_to_bf16_bits(synth.make_tensor(rng, (M, K), "t3"))
    X[:, :16] = synth.f32_to_bf16_bits(synth.make_tensor(rng, (M, 16), "normal", 1e3))  # wide exponent range
    Wa = synth.f32_to_bf16_bits(synth.make_tensor(rng, (ra, K), "normal", 0.05))
    Wb = synth.f32_to_bf16_bits(synth.make_tensor(rng, (rb, K), "normal", 0.01))
    say(f"[quant-lowrank] {M}x{K} ra={ra} rb={rb}")
    x, wa, wb = dev_bf16(X), dev_bf16(Wa), dev_bf16(Wb)
    out, codes, scales = ops.quant_lowrank(x, wa, wb)
    rows = _sample_strips(M, rng) if M > 1024 else np.arange(M)
    c_ref, s_ref = O.quantize_block16(X[rows] if M > 1024 else X, "pow2")
    got_c, got_s = host(codes), host(scales)
    if M > 1024:
        strips = np.unique(rows // 16)
        assert np.array_equal(got_c[rows], O.pack_rm(c_ref))
        assert np.array_equal(got_s[strips], s_ref)
    else:
        assert np.array_equal(got_c, O.pack_rm(c_ref))
        assert np.array_equal(got_s, s_ref)
    if ra + rb:
        assert np.array_equal(host(out), host(ops.lowrank_fused(x, wa, wb)))
        Xf = O.bf16_to_f64(X[rows])
        ref = np.concatenate([Xf @ O.bf16_to_f64(Wa).T, Xf @ O.bf16_to_f64(Wb).T], axis=1)
        assert O.rel_frob(host(out)[rows], ref) < 1e-5


def test_gelu_matches_oracle():
    require_gpu()
    from bit_quantized_lora_amd import ops
    rng = np.random.default_rng(3)
    y = synth.f32_to_bf16_bits((rng.standard_normal(1 << 16) * 3).astype(np.float32))
    dh = synth.f32_to_bf16_bits(rng.standard_normal(1 << 16).astype(np.float32))
    h = host(ops.gelu_fwd(dev_bf16(y)))
    dy = host(ops.gelu_bwd(dev_bf16(y), dev_bf16(dh)))
    yv = O.bf16_to_f64(y)
    ref_h = O.f64_to_bf16_bits(O.gelu(yv))
    ref_dy = O.f64_to_bf16_bits(O.gelu_grad(yv) * O.bf16_to_f64(dh))
    # fp32 math vs fp64: the bf16 results agree bit for bit except next to a
    # rounding boundary (one bf16 ulp) and in the far negative tail where the
    # value is below ~1e-30 and fp32 underflows (absolute error only)
    for got, ref in ((h, ref_h), (dy, ref_dy)):
        g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
        assert np.mean(got == ref) > 0.99
        assert np.all(np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 1e-30)


def _sample_strips(M, rng, n=6):
    s = np.unique(np.concatenate([[0, M // 16 - 1], rng.integers(0, M // 16, n)]))
    return np.concatenate([np.arange(16 * i, 16 * i + 16) for i in s])


@pytest.mark.parametrize("path", ["codes", "op"])
@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_full_size_configs_sampled_rows(cfg, path):
    """Full-size launches (as the benchmark runs them); Y and dX are checked on
    sampled 16-row strips against the oracle, dA and dB in full."""
    require_gpu()
    for d in synth.config_linears(cfg):
        spec = d["spec"]
        if "X" not in d:  # second linear of a pair: a seeded stand-in input of the same shape
            rng = np.random.default_rng(99)
            d["X"] = synth.f32_to_bf16_bits(synth.make_tensor(rng, (spec.M, spec.K), "t3"))
        say(f"[linear] full {spec.name} M={spec.M} K={spec.K} N={spec.N} rs={spec.rs} r={spec.r} path={path}")
        gpu = _gpu_linear(d, path=path)
        rows = _sample_strips(spec.M, np.random.default_rng(spec.M))
        _compare(gpu, _oracle_rows(d, rows), rows, f"{spec.name}/{path}")


@pytest.mark.parametrize("path", ["codes", "op"])
@pytest.mark.parametrize("K,rs,r", [(384, 16, 16), (1024, 32, 16)], ids=["K384", "K1024"])
def test_wide_tile_ragged_edges(path, K, rs, r):
    """A shape for which the 192 x 384 workgroup tile fills the chip better than
    256 x 256 (so the forward GEMM takes it), with ragged last tiles in both M
    and N; rows sampled across the tiles, including the last ones.  K = 384:
    3 stages (fewer than the ring's depth), K = 1024: 8."""
    require_gpu()
    M, N = 4592, 12272
    rng = np.random.default_rng(4592 + K)
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_dist="t3")
    d = synth.make_linear(spec, rng)
    say(f"[linear] wide-tile ragged M={M} K={K} N={N} rs={rs} r={r} path={path}")
    gpu = _gpu_linear(d, path=path)
    rows = np.unique(np.concatenate([_sample_strips(M, rng, 10), np.arange(M - 48, M)]))
    _compare(gpu, _oracle_rows(d, rows), rows, f"wide-tile/K{K}/{path}")


def test_square_tiles_one_round_ragged():
    """256 x 256 tiles, one workgroup per tile (17 x 13 tiles: fewer than CUs, too
    many rows for the 128 x 128 tile), ragged last tiles in M and N, 8 stages."""
    require_gpu()
    from bit_quantized_lora_amd import ops
    M, K, N = 4112, 1024, 3088
    assert ops.linear_plan(M, N, K) == (256, 256, 1)
    rng = np.random.default_rng(528)
    spec = synth.LinearSpec("t", M, K, N, 16, 16, x_dist="t3")
    d = synth.make_linear(spec, rng)
    say(f"[linear] square tiles, one round, M={M} K={K} N={N}")
    gpu = _gpu_linear(d, path="codes")
    rows = np.unique(np.concatenate([_sample_strips(M, rng, 8), np.arange(M - 48, M)]))
    _compare(gpu, _oracle_rows(d, rows), rows, "square-tile/one-round")


# Big tiles with few stages and many ranks: ragged last tiles in M and N, both
# tile shapes, 3-4 stages, no low-rank term, the largest rank (8 chunks of 16
# ranks), ranks from both factors, and the backward's transposed GEMM.
BIG_EDGES = [
    # (M, K, N, rs, r)
    (4624, 384, 4624, 16, 0),
    (4624, 384, 4624, 64, 64),
    (4624, 512, 4624, 0, 0),
    (4624, 512, 4624, 48, 16),
    (4592, 384, 12272, 64, 64),
    (4624, 4624, 512, 16, 16),     # the dX GEMM reduces over 512: pipelined, square tiles
]


@pytest.mark.parametrize("case", BIG_EDGES, ids=lambda c: "x".join(map(str, c)))
def test_big_tile_edges(case):
    require_gpu()
    from bit_quantized_lora_amd import ops
    M, K, N, rs, r = case
    say(f"[linear] big tiles {case}: fwd plan {ops.linear_plan(M, N, K)}, backward plan "
        f"{ops.linear_bwd_plan(M, N, K, r)}")
    rng = np.random.default_rng(M + K + N + rs)
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_outlier_frac=0.01, x_outlier_mult=50.0)
    d = synth.make_linear(spec, rng)
    gpu = _gpu_linear(d)
    rows = np.unique(np.concatenate([_sample_strips(M, rng, 10), np.arange(M - 48, M)]))
    _compare(gpu, _oracle_rows(d, rows), rows, f"big-tiles{case}")


# Few tokens: the 512 text tokens of a FLUX block (configuration 5's text-stream
# linears, whole), and ragged variants.  Fewer 256 x 256 tiles than compute
# units, so the GEMMs take 128 x 128 tiles and, where the reduction is long,
# split it (fp32 partial products summed in split order by a second kernel).
SMALL_M = [
    # (M, K, N, rs, r)
    (512, 3072, 9216, 32, 32),      # qkv
    (512, 3072, 3072, 32, 32),      # out-proj
    (512, 3072, 12288, 32, 32),     # MLP up
    (512, 12288, 3072, 32, 32),     # MLP down
    (400, 3072, 1040, 16, 16),      # ragged last tiles in M and N
    (272, 4224, 656, 32, 16),       # ragged, 33 stages (uneven splits)
    (528, 5248, 1040, 16, 16),      # ragged, 41 stages
]


def _small_m_data(shape):
    M, K, N, rs, r = shape
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_outlier_frac=0.01, x_outlier_mult=50.0)
    return synth.make_linear(spec, np.random.default_rng(M + 3 * K + 7 * N))


@pytest.mark.parametrize("shape", SMALL_M, ids=lambda s: "x".join(map(str, s)))
def test_small_m_tiles_and_split_reduction(shape):
    """Every element of Y, dX, dA, dB against the oracle; the forward without a
    workspace (never split) agrees as well; a split forward repeated gives the
    same bits."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, K, N, rs, r = shape
    fwd, fwd_nows, bwd = ops.linear_plan(M, N, K), ops.linear_plan(M, N, K, with_ws=False), \
        ops.linear_bwd_plan(M, N, K, r)
    say(f"[linear] few tokens {shape}: fwd plan {fwd} (no workspace {fwd_nows}), dX plan {bwd}")
    assert fwd[:2] == (128, 128) and fwd_nows == (128, 128, 1)
    d = _small_m_data(shape)
    gpu = _gpu_linear(d)
    rows = np.arange(M)
    _compare(gpu, _oracle_rows(d, rows), rows, f"few-tokens{shape}")
    # the same forward through ft_linear_fwd (no workspace, whole reduction per tile)
    X, R = dev_bf16(d["X"]), dev_bf16(d["R"])
    L1t, At = dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(np.ascontiguousarray(d["A"].T))
    L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
    xq, _, xs = ops.quant_block16(X)
    rq, _, rsc = ops.quant_block16(R)
    T = ops.lowrank_fused(X, L1t, At)
    Y1 = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K, split=False)
    Y2 = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K)
    Y3 = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K)
    torch.cuda.synchronize()
    ref = _oracle_rows(d, rows)["Y"]
    e1 = O.rel_frob(host(Y1).astype(np.float64), ref)
    say(f"[linear] few tokens {shape}: unsplit forward rel-Frobenius {e1:.2e}")
    assert e1 <= BUDGET
    assert np.array_equal(host(Y2).view(np.uint32), host(Y3).view(np.uint32)), "split forward not deterministic"
    if fwd[2] == 1:
        assert np.array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))


def test_small_m_set_covers_split_paths():
    """The few-token shapes above take both the split and the unsplit small-tile
    GEMM, forward and backward (as planned for this device's compute units)."""
    require_gpu()
    from bit_quantized_lora_amd import ops
    fwd = [ops.linear_plan(M, N, K) for M, K, N, _, _ in SMALL_M]
    bwd = [ops.linear_bwd_plan(M, N, K, r)[:3] for M, K, N, _, r in SMALL_M]
    say(f"[linear] few-token plans: fwd {fwd}, dX {bwd}")
    assert any(p[2] > 1 for p in fwd) and any(p[2] == 1 for p in fwd)
    assert any(p[2] > 1 for p in bwd) and any(p[:2] == (128, 128) and p[2] == 1 for p in bwd)


@pytest.mark.parametrize("shape", [(272, 384, 512), (304, 1040, 400)], ids=lambda s: "x".join(map(str, s)))
def test_op_path_with_unmerged_pairs_in_both_operands(shape):
    """Outlier columns x2000 in X and in W open exponent gaps beyond the E3M2
    range in both GEMM operands (forward: X and R; backward: G and R^T), so
    k-steps take the two-round MFMA path; results stay within the budget and
    match the codes path."""
    require_gpu()
    import torch
    M, K, N = shape
    rng = np.random.default_rng(K + N)
    spec = synth.LinearSpec("t", M, K, N, 16, 16, x_outlier_count=8, x_outlier_mult=2000.0,
                            w_outlier_cols=8, w_outlier_mult=2000.0)
    d = synth.make_linear(spec, rng)
    # G with outlier output channels, so the backward's left operand is split too;
    # R with outlier columns and rows (the stabilizer split absorbs W's outlier
    # columns, so R is scaled directly: any bf16 R is a valid GEMM input)
    G = synth.bf16_bits_to_f32(d["G"])
    G[:, rng.choice(N, 8, replace=False)] *= np.float32(2000.0)
    d["G"] = synth.f32_to_bf16_bits(G)
    R = synth.bf16_bits_to_f32(d["R"])
    R[:, rng.choice(K, 8, replace=False)] *= np.float32(2000.0)
    R[rng.choice(N, 8, replace=False), :] *= np.float32(2000.0)
    d["R"] = synth.f32_to_bf16_bits(R)
    for name, bits in (("X", d["X"]), ("R", d["R"]), ("G", d["G"]), ("R^T", np.ascontiguousarray(d["R"].T))):
        c, sc = O.quantize_block16(bits)
        _, osc = O.operand_merge(c, sc)
        assert np.any(osc[:, 0::2] != osc[:, 1::2]), f"{name}: expected unmerged pairs"
    say(f"[linear] unmerged pairs {shape}")
    gpu = _gpu_linear(d, path="op")
    rows = np.arange(M)
    _compare(gpu, _oracle_rows(d, rows), rows, f"unmerged{shape}")
    ref = _gpu_linear(d, path="codes")
    for k in ("Y", "dX", "dA", "dB"):
        assert O.rel_frob(host(gpu[k]), host(ref[k]).astype(np.float64)) < 1e-5


@pytest.mark.parametrize("case", [(144, 400, 16, 16), (528, 1040, 32, 32), (272, 256, 0, 64), (4608, 12288, 32, 16),
                                  (48, 128, 64, 64)], ids=lambda c: "x".join(map(str, c)))
def test_quant_lowrank_db_folds_the_adapter_gradient(case):
    """The backward's pass over G with dB = (X A)^T G folded in: codes and scales
    bit-identical to ft_quant_lowrank, V equal to it up to fp32 summation order
    (this pass keeps 128-row blocks, ft_quant_lowrank adds two column groups per
    64-row block), dB within fp32 rounding of the oracle's fp64 product."""
    require_gpu()
    import torch
    from bit_quantized_lora_amd import ops
    M, N, rs, r = case
    rng = np.random.default_rng(M + N + r)
    G = synth.f32_to_bf16_bits(synth.make_tensor(rng, (M, N), "normal", 1e-3))
    L2 = synth.f32_to_bf16_bits(synth.make_tensor(rng, (rs, N), "normal", 0.05))
    B = synth.f32_to_bf16_bits(synth.make_tensor(rng, (r, N), "normal", 0.01))
    T = synth.make_tensor(rng, (M, rs + r), "t3").astype(np.float32)
    say(f"[quant-lowrank-db] M={M} N={N} rs={rs} r={r}")
    g, l2, b = dev_bf16(G), dev_bf16(L2), dev_bf16(B)
    t = torch.from_numpy(T).cuda()
    V, codes, scales, dB = ops.quant_lowrank_db(g, l2, b, t)
    V0, codes0, scales0 = ops.quant_lowrank(g, l2, b)
    torch.cuda.synchronize()
    assert O.rel_frob(host(V).astype(np.float64), host(V0).astype(np.float64)) < 1e-6
    assert np.array_equal(host(codes), host(codes0)) and np.array_equal(host(scales), host(scales0))
    ref = T[:, rs:].astype(np.float64).T @ O.bf16_to_f64(G)
    assert O.rel_frob(host(dB).astype(np.float64), ref) < 1e-5
