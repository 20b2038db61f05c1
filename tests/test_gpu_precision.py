"""Parity of the precision variants (FourTune section 4.3, "Impact of Precision
Configurations", Table 4) against the fp64 CPU oracle.

W4A16: the forward backbone product takes the bf16 activations unquantized (the
oracle's Eq. 2 with X for Q(X)); G16: the backward product takes the bf16 output
gradient unquantized (Eq. 3 with G for Q(G)).  R stays quantized with the same
Q(.) as in W4A4G4.  The GPU product runs on bf16 MFMA with Q(R) dequantized to
bf16, which is exact for every block scale above 2^-126, and accumulates in fp32:
the same contract (relative Frobenius <= 2e-3) and fp32 budget (1e-4) as the
W4A4G4 calls.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
BUDGET = 1e-4


def _gpu_variant(d, a16: bool, g16: bool, out_dtype=None):
    """Forward and backward of one linear with the chosen operand precisions."""
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
    rq, rqc, rsc, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
    if a16:
        Y = ops.linear_fwd_a16(X, rq, rsc, T, L2, B, M, N, K, out_dtype=out_dtype)
    else:
        xq, _, xs = ops.quant_block16(X)
        Y = ops.linear_fwd(xq, xs, rq, rsc, T, L2, B, M, N, K, out_dtype=out_dtype)
    if g16:
        dX, dAt, dB = ops.linear_bwd_g16(G, rqc, rsct, V, L1t, At, X, T, M, N, K, out_dtype=out_dtype)
    else:
        gq, _, gs = ops.quant_block16(G)
        dX, dAt, dB = ops.linear_bwd(gq, gs, rqc, rsct, V, L1t, At, X, G, T, M, N, K, out_dtype=out_dtype)
    return {"Y": Y, "dX": dX, "dA": dAt, "dB": dB}


def _oracle_variant(d, rows, a16: bool, g16: bool):
    """Oracle Y and dX on `rows` (16-row strips) with X / G unquantized where
    the variant says so; full dA, dB."""
    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "R", "L1", "L2", "A", "B", "G")}
    rc, rsc = O.quantize_block16(d["R"])
    Rhat = O.dequantize(rc, rsc, "pow2")
    Xr, Gr = f["X"][rows], f["G"][rows]
    if a16:
        Xhat = Xr
    else:
        xc, xs = O.quantize_block16(d["X"][rows])
        Xhat = O.dequantize(xc, xs, "pow2")
    if g16:
        Ghat = Gr
    else:
        gc, gs = O.quantize_block16(d["G"][rows])
        Ghat = O.dequantize(gc, gs, "pow2")
    Y = O.linear_fwd(Xhat, Rhat, Xr, f["L1"], f["L2"], f["A"], f["B"])
    g = O.linear_bwd(Ghat, Rhat, Gr, Xr, f["L1"], f["L2"], f["A"], f["B"])
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
    say(f"[precision] {label} rel-Frobenius errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL, f"{label}: {k} error {e:.3e} above the 2e-3 contract"
        assert e <= BUDGET, f"{label}: {k} error {e:.3e} above the fp32 precision budget"


def _sample_strips(M, rng, n=6):
    s = np.unique(np.concatenate([[0, M // 16 - 1], rng.integers(0, M // 16, n)]))
    return np.concatenate([np.arange(16 * i, 16 * i + 16) for i in s])


SMALL = [
    # (M, K, N, rs, r): single and several 256-tiles, ragged M / N tails, reduction
    # lengths with a half last stage (K or N % 32 == 16, forward and backward),
    # 1 .. 33 stages, rank edge cases (none, one pass, two low-rank passes)
    (256, 256, 256, 16, 16),
    (144, 400, 272, 16, 16),
    (528, 176, 48, 32, 0),
    (48, 48, 48, 0, 16),
    (80, 528, 304, 64, 64),
    (16, 16, 16, 0, 0),
    (272, 1040, 528, 32, 32),
    (304, 1152, 384, 16, 16),
    (32, 16, 32, 16, 16),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_w4a16g16_small_and_ragged(shape):
    require_gpu()
    M, K, N, rs, r = shape
    rng = np.random.default_rng(M * 5 + K * 3 + N)
    spec = synth.LinearSpec("t", M, K, N, rs, r, x_outlier_count=min(4, K), x_outlier_mult=30.0,
                            w_outlier_cols=min(2, K), w_outlier_mult=20.0)
    d = synth.make_linear(spec, rng)
    say(f"[precision] W4A16G16 small {shape}")
    gpu = _gpu_variant(d, a16=True, g16=True)
    rows = np.arange(M)
    _compare(gpu, _oracle_variant(d, rows, True, True), rows, f"W4A16G16{shape}")


@pytest.mark.parametrize("a16,g16", [(True, False), (False, True)], ids=["W4A16G4", "W4A4G16"])
def test_mixed_settings_small(a16, g16):
    """The two mixed settings of the table: one new product beside one W4A4G4
    product, each against its own oracle."""
    require_gpu()
    M, K, N = 272, 400, 528
    d = synth.make_linear(synth.LinearSpec("t", M, K, N, 32, 16, x_dist="t3"), np.random.default_rng(11))
    gpu = _gpu_variant(d, a16, g16)
    rows = np.arange(M)
    _compare(gpu, _oracle_variant(d, rows, a16, g16), rows, f"a16={a16} g16={g16}")


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_w4a16g16_full_size_sampled_rows(cfg):
    """Full-size launches of the benchmark shapes; Y and dX on sampled 16-row
    strips, dA and dB in full."""
    require_gpu()
    for d in synth.config_linears(cfg):
        spec = d["spec"]
        if "X" not in d:
            d["X"] = synth.f32_to_bf16_bits(synth.make_tensor(np.random.default_rng(99), (spec.M, spec.K), "t3"))
        say(f"[precision] W4A16G16 full {spec.name} M={spec.M} K={spec.K} N={spec.N} rs={spec.rs} r={spec.r}")
        gpu = _gpu_variant(d, True, True)
        rows = _sample_strips(spec.M, np.random.default_rng(spec.M + 1))
        _compare(gpu, _oracle_variant(d, rows, True, True), rows, f"{spec.name}/W4A16G16")


def test_ragged_tiles_at_scale():
    """Ragged last tiles in both M and N of a many-tile launch (forward N =
    12272, backward N = K = 3056), rows sampled across the tiles and the last
    ones."""
    require_gpu()
    M, K, N = 4592, 3056, 12272
    rng = np.random.default_rng(4592)
    d = synth.make_linear(synth.LinearSpec("t", M, K, N, 32, 16, x_dist="t3"), rng)
    say(f"[precision] ragged at scale M={M} K={K} N={N}")
    gpu = _gpu_variant(d, True, True)
    rows = np.unique(np.concatenate([_sample_strips(M, rng, 10), np.arange(M - 48, M)]))
    _compare(gpu, _oracle_variant(d, rows, True, True), rows, "ragged-at-scale")


def test_determinism_and_bf16_outputs():
    require_gpu()
    import torch
    d = synth.config_linears("c1")[0]
    a = _gpu_variant(d, True, True)
    b = _gpu_variant(d, True, True)
    for k in ("Y", "dX", "dA", "dB"):
        assert np.array_equal(host(a[k]).view(np.uint32), host(b[k]).view(np.uint32)), k
    h = _gpu_variant(d, True, True, out_dtype=torch.bfloat16)
    for k in ("Y", "dX"):
        assert np.array_equal(host(h[k]), synth.f32_to_bf16_bits(host(a[k]))), k


def _scaled_case(row_scale: dict, g_cols, seed=5):
    """M = 64, K = 256, N = 64 linear whose R rows 16i .. 16i+15 are scaled by
    row_scale[i] (powers of two) and whose G is zero outside columns g_cols; no
    low-rank terms."""
    M, K, N = 64, 256, 64
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    R = rng.standard_normal((N, K)).astype(np.float32)
    for i, sc in row_scale.items():
        R[16 * i:16 * i + 16] *= np.float32(sc)
    G = np.zeros((M, N), np.float32)
    G[:, g_cols] = rng.standard_normal((M, len(g_cols))).astype(np.float32)
    d = {"X": synth.f32_to_bf16_bits(X), "R": synth.f32_to_bf16_bits(R), "G": synth.f32_to_bf16_bits(G)}
    for k, shp in (("L1", (K, 16)), ("L2", (16, N)), ("A", (K, 16)), ("B", (16, N))):
        d[k] = np.zeros(shp, np.uint16)
    return d


def _check_strips(gpu, ref, label):
    """Y per 16-column strip (each strip is one R row block, one scale range)
    and dX whole, so that a lost or mis-scaled block cannot hide under the norm
    of a larger one."""
    got = host(gpu["Y"]).astype(np.float64)
    for c0 in range(0, got.shape[1], 16):
        e = O.rel_frob(got[:, c0:c0 + 16], ref["Y"][:, c0:c0 + 16])
        assert e <= BUDGET, f"{label}: Y columns {c0}..{c0 + 15}: {e:.3e}"
    e = O.rel_frob(host(gpu["dX"]).astype(np.float64), ref["dX"])
    assert e <= BUDGET, f"{label}: dX {e:.3e}"


@pytest.mark.parametrize("g_block", [0, 3], ids=["tiny", "huge"])
def test_extreme_block_scales(g_block):
    """R row blocks at the ends of the scale range (E about -124 and +120: the
    dequantized values are normal bf16 numbers), next to ordinary blocks.  The
    forward checks every block; the backward takes G nonzero only on the output
    columns of the tiny (or huge) block, so dX is that block's product alone."""
    require_gpu()
    d = _scaled_case({0: 2.0 ** -122, 1: 1.0, 2: 2.0 ** -60, 3: 2.0 ** 120},
                     list(range(16 * g_block, 16 * g_block + 16)))
    _, sc = O.quantize_block16(d["R"])
    assert sc[0].max() <= 127 - 119 and sc[3].min() >= 127 + 119
    say(f"[precision] extreme block scales, backward through block {g_block}")
    gpu = _gpu_variant(d, True, True)
    _check_strips(gpu, _oracle_variant(d, np.arange(64), True, True), f"extreme/{g_block}")
