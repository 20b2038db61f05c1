"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against the format definition, a
brute-force search in exact rational arithmetic, a closed form, an
invariant or a special case that reduces to a textbook computation.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = (b >> 7) & 0xFF
    return b[expo != 0xFF]


# ---------------------------------------------------------------- E2M1 decode
def test_e2m1_decode_matches_published_table():
    rows = _read_golden("e2m1_table.txt")
    assert len(rows) == 16
    for bits, val in rows:
        code = int(bits, 2)
        got = O.e2m1_decode(np.array([code]))[0]
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


# ---------------------------------------------------------------- RNE
_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
         Fraction(3), Fraction(4), Fraction(6)]


def _rne_bruteforce(v: float) -> int:
    """Nearest E2M1 magnitude by exact rational distance; ties to the even code."""
    a = abs(Fraction(v))
    if a > 6:
        idx = 7
    else:
        d = [abs(a - g) for g in _GRID]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
    sign = 1 if math.copysign(1.0, v) < 0 else 0
    return (sign << 3) | idx


def test_rne_hand_worked_cases():
    for v, bits in _read_golden("e2m1_rne_cases.txt"):
        got = int(O.e2m1_rne(np.array([float(v)]))[0])
        assert got == int(bits, 2), (v, got, bits)


def test_rne_exhaustive_bf16_ratios():
    """Every finite bf16 value, as a ratio, against exact-rational brute force."""
    vals = O.bf16_to_f64(_all_finite_bf16())
    got = O.e2m1_rne(vals)
    # brute force on the distinct magnitudes, then apply sign
    mags = np.unique(np.abs(vals))
    table = {float(m): _rne_bruteforce(float(m)) for m in mags}
    exp = np.array([table[abs(float(v))] | (8 if math.copysign(1, v) < 0 else 0)
                    for v in vals], dtype=np.uint8)
    assert np.array_equal(got, exp)


def test_rne_fp32_neighbourhood_of_midpoints():
    """fp32 ratios (the "f32" scale rule produces them) next to every midpoint."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 3.0],
                    dtype=np.float32)
    vals = []
    for m in mids:
        x = np.float32(m)
        lo = x; hi = x
        for _ in range(4):
            vals += [lo, hi]
            lo = np.nextafter(lo, np.float32(0)); hi = np.nextafter(hi, np.float32(10))
    rng = np.random.default_rng(3)
    vals += list(rng.uniform(0, 7, 3000).astype(np.float32))
    vals = np.array(vals, dtype=np.float32).astype(np.float64)
    vals = np.concatenate([vals, -vals])
    got = O.e2m1_rne(vals)
    exp = np.array([_rne_bruteforce(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, exp)


# ---------------------------------------------------------------- scales
def _pow2_bruteforce(amax: Fraction) -> int:
    """Smallest integer e with 6 * 2^e >= amax, clamped to [-127, 127], by bisection."""
    if amax == 0:
        return -127
    lo, hi = -300, 300          # 6*2^lo < amax <= 6*2^hi
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if 6 * Fraction(2) ** mid >= amax:
            hi = mid
        else:
            lo = mid
    return max(-127, min(127, hi))


def test_scale_pow2_exhaustive():
    b = _all_finite_bf16()
    b = b[b < 0x8000]                       # non-negative amax values
    vals = O.bf16_to_f64(b)
    got = O.scale_pow2_exponent(vals)
    exp = np.array([_pow2_bruteforce(Fraction(float(v))) for v in vals])
    assert np.array_equal(got, exp)
    # no element of a block can saturate: amax * 2^-E <= 6, and E is minimal
    nz = (vals > 0) & (exp > -127)
    assert np.all(vals[nz] * np.exp2(-exp[nz]) <= 6.0)
    assert np.all(vals[nz] * np.exp2(-(exp[nz] - 1.0)) > 6.0)


def _fp32_round_exact(q: Fraction) -> np.float32:
    """Correctly rounded binary32 of a positive rational, by checking neighbours."""
    approx = np.float32(float(q))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)),
             np.nextafter(approx, np.float32(0))}
    cands = sorted(float(c) for c in cands)
    best = None
    for c in cands:
        d = abs(Fraction(c) - q)
        if best is None or d < best[0]:
            best = (d, [c])
        elif d == best[0]:
            best[1].append(c)
    if len(best[1]) == 1:
        return np.float32(best[1][0])
    for c in best[1]:           # tie: even mantissa (last bit of the binary32 pattern 0)
        if int(np.float32(c).view(np.uint32)) % 2 == 0:
            return np.float32(c)
    raise AssertionError


def test_scale_f32_exhaustive():
    b = _all_finite_bf16()
    b = b[b < 0x8000]
    vals = O.bf16_to_f64(b)
    got = O.scale_f32(vals)
    exp = np.array([_fp32_round_exact(Fraction(float(v)) / 6) if v > 0 else np.float32(0)
                    for v in vals], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


# ---------------------------------------------------------------- quantizer
def _blocks_from_codes(rng, br, bc, mode):
    """Blocks c * s with representable codes, each block holding a code of magnitude 4 or 6."""
    codes = rng.integers(0, 16, size=(br * 16, bc * 16)).astype(np.uint8)
    for i in range(br):
        for j in range(bc):
            codes[16 * i + rng.integers(16), 16 * j + rng.integers(16)] = rng.choice([6, 7, 14, 15])
            if mode == "f32":
                codes[16 * i + rng.integers(16), 16 * j + rng.integers(16)] = rng.choice([7, 15])
    vals = O.e2m1_decode(codes)
    if mode == "pow2":
        E = rng.integers(-120, 120, size=(br, bc))
        s = np.exp2(E.astype(np.float64))
        scales = (E + 127).astype(np.uint8)
    else:
        # s = 1.25 * 2^k: 6 s and every c * s fit in bf16; fl32(6 s / 6) = s
        k = rng.integers(-60, 60, size=(br, bc))
        s = 1.25 * np.exp2(k.astype(np.float64))
        scales = s.astype(np.float32)
    x = vals * np.repeat(np.repeat(s, 16, 0), 16, 1)
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(O.bf16_to_f64(bits), x)   # exactly representable
    return bits, codes, scales


@pytest.mark.parametrize("mode", ["pow2", "f32"])
def test_quantizer_roundtrip_of_representable_blocks(mode):
    rng = np.random.default_rng(11)
    bits, codes, scales = _blocks_from_codes(rng, 4, 6, mode)
    got_codes, got_scales = O.quantize_block16(bits, mode)
    # a zero code carries the sign of the zero it came from; compare values for those
    nz = (codes & 7) != 0
    assert np.array_equal(got_codes[nz], codes[nz])
    assert np.all((got_codes[~nz] & 7) == 0)
    if mode == "pow2":
        assert np.array_equal(got_scales, scales)
    else:
        assert np.array_equal(got_scales.view(np.uint32), scales.view(np.uint32))
    assert np.array_equal(O.dequantize(got_codes, got_scales, mode), O.bf16_to_f64(bits))


@pytest.mark.parametrize("mode", ["pow2", "f32"])
def test_quantizer_elementwise_bruteforce(mode):
    """Small random tensor, every element re-derived by exact rational brute force."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((32, 48)) * np.exp2(rng.integers(-4, 4, (32, 48)))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    codes, scales = O.quantize_block16(bits, mode)
    xv = O.bf16_to_f64(bits)
    for bi in range(2):
        for bj in range(3):
            blk = xv[16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16]
            amax = Fraction(float(np.abs(blk).max()))
            if mode == "pow2":
                E = _pow2_bruteforce(amax)
                assert scales[bi, bj] == E + 127
                ratio = lambda v: float(Fraction(v) / Fraction(2) ** E)
            else:
                s = _fp32_round_exact(amax / 6)
                assert scales[bi, bj] == s
                ratio = lambda v: float(_fp32_round_exact(abs(Fraction(v)) / Fraction(float(s)))) * \
                    (1 if math.copysign(1, v) > 0 else -1) if v != 0 else v
            for i in range(16):
                for j in range(16):
                    v = float(blk[i, j])
                    exp = _rne_bruteforce(ratio(v))
                    assert codes[16 * bi + i, 16 * bj + j] == exp


@pytest.mark.parametrize("kind", ["zeros", "negzeros", "subnormal", "ties", "huge", "mixed"])
@pytest.mark.parametrize("mode", ["pow2", "f32"])
def test_quantizer_edge_invariants(kind, mode):
    bits = synth.edge_tensor(kind, 64, 64)
    codes, scales = O.quantize_block16(bits, mode)
    x = O.bf16_to_f64(bits)
    xhat = O.dequantize(codes, scales, mode)
    # sign bit follows the input's sign bit
    assert np.array_equal((codes >> 3).astype(bool), np.signbit(x))
    # each element lands on one of the two grid neighbours of its ratio
    s = np.repeat(np.repeat(O.scale_values(scales, mode), 16, 0), 16, 1)
    with np.errstate(all="ignore"):
        err = np.where(s > 0, np.abs(xhat - x) / np.where(s > 0, s, 1), 0.0)
    # half a grid step is at most 1 (between 4 and 6); saturation is absent for pow2
    assert np.all(err <= 1.0 + 1e-12)
    if kind in ("zeros", "negzeros"):
        assert np.all((codes & 7) == 0)
        if mode == "pow2":
            assert np.all(scales == 0)
        else:
            assert np.all(scales == 0)


def test_transposition_invariance():
    """The same 16x16 blocks serve Q(R) and Q(R)^T (section 3.2)."""
    rng = np.random.default_rng(9)
    for mode in ("pow2", "f32"):
        bits = synth.f32_to_bf16_bits(rng.standard_t(3, (48, 80)).astype(np.float32))
        c, s = O.quantize_block16(bits, mode)
        ct, st = O.quantize_block16(np.ascontiguousarray(bits.T), mode)
        assert np.array_equal(ct, c.T)
        assert np.array_equal(np.asarray(st), np.asarray(s).T)
        assert np.array_equal(O.pack_cm(c), O.pack_rm(ct))


def test_packing_layout():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, (16, 32)).astype(np.uint8)
    rm = O.pack_rm(c)
    cm = O.pack_cm(c)
    flat_rm = np.zeros(16 * 32 // 2, np.uint8)
    flat_cm = np.zeros(16 * 32 // 2, np.uint8)
    for i in range(16):
        for j in range(32):
            idx = i * 32 + j
            flat_rm[idx // 2] |= c[i, j] << (4 * (idx % 2))
            idx = j * 16 + i
            flat_cm[idx // 2] |= c[i, j] << (4 * (idx % 2))
    assert np.array_equal(rm.reshape(-1), flat_rm)
    assert np.array_equal(cm.reshape(-1), flat_cm)
    assert np.array_equal(O.unpack_rm(rm, 32), c)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rounding_agrees_with_integer_rne():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.exp2(rng.integers(-140, 120, 200000)).astype(np.float32),
        (np.arange(1, 5000, dtype=np.uint32) << 15 | 0x3F800000).view(np.float32),  # exact halfway cases
    ])
    x = x[np.isfinite(x)]
    a = O.f64_to_bf16_bits(x.astype(np.float64))
    b = synth.f32_to_bf16_bits(x)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- linear algebra
def _frac_mat(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a)]


def _frac_mm(a, b):
    n, k, m = len(a), len(b), len(b[0])
    return [[sum(a[i][t] * b[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def _frac_T(a):
    return [list(r) for r in zip(*a)]


def _frac_add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def _tiny_linear(M, K, N, rs, r, seed):
    rng = np.random.default_rng(seed)
    spec = synth.LinearSpec("tiny", M, K, N, rs, r)
    d = synth.make_linear(spec, rng)
    f = {k: O.bf16_to_f64(d[k]) for k in ("X", "W", "R", "L1", "L2", "A", "B", "G")}
    xc, xs = O.quantize_block16(d["X"]); rc, rsc = O.quantize_block16(d["R"])
    gc, gs = O.quantize_block16(d["G"])
    f["Xhat"] = O.dequantize(xc, xs, "pow2")
    f["Rhat"] = O.dequantize(rc, rsc, "pow2")
    f["Ghat"] = O.dequantize(gc, gs, "pow2")
    return f


@pytest.mark.parametrize("shape", [(16, 16, 16, 2, 3), (32, 64, 48, 4, 4)])
def test_linear_fwd_bwd_exact_rational(shape):
    M, K, N, rs, r = shape
    f = _tiny_linear(M, K, N, rs, r, 21)
    Y = O.linear_fwd(f["Xhat"], f["Rhat"], f["X"], f["L1"], f["L2"], f["A"], f["B"])
    g = O.linear_bwd(f["Ghat"], f["Rhat"], f["G"], f["X"], f["L1"], f["L2"], f["A"], f["B"])
    F = {k: _frac_mat(v) for k, v in f.items()}
    # Eq. 2 term by term in exact arithmetic, with R in out x in layout
    Yq = _frac_mm(F["Xhat"], _frac_T(F["Rhat"]))
    Ys = _frac_mm(F["X"], _frac_mm(F["L1"], F["L2"]))
    Ya = _frac_mm(_frac_mm(F["X"], F["A"]), F["B"])
    Yx = _frac_add(_frac_add(Yq, Ys), Ya)
    dXq = _frac_mm(F["Ghat"], F["Rhat"])
    dXs = _frac_mm(_frac_mm(F["G"], _frac_T(F["L2"])), _frac_T(F["L1"]))
    dXa = _frac_mm(_frac_mm(F["G"], _frac_T(F["B"])), _frac_T(F["A"]))
    dXx = _frac_add(_frac_add(dXq, dXs), dXa)
    dBx = _frac_mm(_frac_T(_frac_mm(F["X"], F["A"])), F["G"])
    dAx = _frac_mm(_frac_T(F["X"]), _frac_mm(F["G"], _frac_T(F["B"])))
    for got, ex in ((Y, Yx), (g["dX"], dXx), (g["dB"], dBx), (g["dA"], dAx)):
        ex = np.array([[float(v) for v in row] for row in ex])
        assert O.rel_frob(got, ex) < 1e-14


def test_linear_special_cases_reduce_to_plain_gemm():
    """With Q-representable X, R, G the triple-branch layer is one dense layer
    with weight W' = R + (L1 L2)^T + (A B)^T (out x in)."""
    rng = np.random.default_rng(4)
    M, K, N, rs, r = 48, 64, 32, 3, 5
    def representable(rows, cols):
        b, _, _ = _blocks_from_codes(rng, rows // 16, cols // 16, "pow2")
        return b
    X, R, G = representable(M, K), representable(N, K), representable(M, N)
    Xf, Rf, Gf = (O.bf16_to_f64(t) for t in (X, R, G))
    L1 = rng.standard_normal((K, rs)); L2 = rng.standard_normal((rs, N))
    A = rng.standard_normal((K, r)); B = rng.standard_normal((r, N))
    for t, f in ((X, Xf), (R, Rf), (G, Gf)):
        c, s = O.quantize_block16(t)
        assert np.array_equal(O.dequantize(c, s, "pow2"), f)
    Wp = Rf + (L1 @ L2).T + (A @ B).T
    Y = O.linear_fwd(Xf, Rf, Xf, L1, L2, A, B)
    assert O.rel_frob(Y, Xf @ Wp.T) < 1e-14
    g = O.linear_bwd(Gf, Rf, Gf, Xf, L1, L2, A, B)
    assert O.rel_frob(g["dX"], Gf @ Wp) < 1e-14
    # no low-rank branches: pure W4A4 GEMM; zero residual: pure low-rank layer
    z = np.zeros
    assert O.rel_frob(O.linear_fwd(Xf, Rf, Xf, z((K, 0)), z((0, N)), z((K, 0)), z((0, N))), Xf @ Rf.T) < 1e-15
    Y0 = O.linear_fwd(Xf, z((N, K)), Xf, L1, L2, A, B)
    assert O.rel_frob(Y0, Xf @ (L1 @ L2 + A @ B)) < 1e-14


def test_adapter_gradients_finite_differences():
    """dA, dB are the exact gradients of L = <G, Y(A, B)> (section 3.2)."""
    rng = np.random.default_rng(8)
    M, K, N, r = 32, 16, 24, 4
    X = rng.standard_normal((M, K)); G = rng.standard_normal((M, N))
    A = rng.standard_normal((K, r)); B = rng.standard_normal((r, N))
    z = np.zeros
    def loss(A_, B_):
        Y = O.linear_fwd(z((M, K)), z((N, K)), X, z((K, 0)), z((0, N)), A_, B_)
        return float(np.sum(G * Y))
    g = O.linear_bwd(z((M, N)), z((N, K)), G, X, z((K, 0)), z((0, N)), A, B)
    h = 1e-5
    for name, P, grad in (("A", A, g["dA"]), ("B", B, g["dB"])):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            Pp = P.copy(); Pm = P.copy()
            Pp[idx] += h; Pm[idx] -= h
            args_p = (Pp, B) if name == "A" else (A, Pp)
            args_m = (Pm, B) if name == "A" else (A, Pm)
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert O.rel_frob(grad, fd) < 1e-8


def test_input_gradient_finite_differences_straight_through():
    """dX of Eq. 3 equals d<G, Y>/dX when Q acts as identity and G is representable."""
    rng = np.random.default_rng(12)
    M, K, N, rs, r = 16, 32, 16, 2, 3
    X = rng.standard_normal((M, K))
    Rf = rng.standard_normal((N, K)); L1 = rng.standard_normal((K, rs)); L2 = rng.standard_normal((rs, N))
    A = rng.standard_normal((K, r)); B = rng.standard_normal((r, N))
    G = rng.standard_normal((M, N))
    loss = lambda X_: float(np.sum(G * O.linear_fwd(X_, Rf, X_, L1, L2, A, B)))
    g = O.linear_bwd(G, Rf, G, X, L1, L2, A, B)
    h = 1e-5
    fd = np.zeros_like(X)
    for idx in np.ndindex(X.shape):
        Xp = X.copy(); Xm = X.copy(); Xp[idx] += h; Xm[idx] -= h
        fd[idx] = (loss(Xp) - loss(Xm)) / (2 * h)
    assert O.rel_frob(g["dX"], fd) < 1e-8


# ---------------------------------------------------------------- GELU
# Phi(x) to 40+ significant digits, computed here from two textbook series in
# decimal arithmetic (independent of scipy, which the oracle calls):
#  * Maclaurin series of erf, Phi(x) = 1/2 + erf(x / sqrt 2) / 2, with enough
#    working digits to survive the cancellation far in the lower tail;
#  * Laplace's continued fraction for the Mills ratio, Phi(-x) = phi(x) R(x) with
#    R(x) = 1/(x + 1/(x + 2/(x + 3/(x + ...)))), for x >= 5.
# The two agree to 35 digits where both apply, which pins each of them.
def _dec_pi(ctx):
    from decimal import Decimal
    def arctan_inv(n):   # arctan(1/n) by its Taylor series
        x = Decimal(1) / n; x2 = x * x; t = x; s = x; k = 1
        while True:
            t *= -x2; k += 2
            d = t / k
            if abs(d) < Decimal(10) ** (-ctx.prec - 2):
                return s
            s += d
    return 16 * arctan_inv(5) - 4 * arctan_inv(239)   # Machin


def _phi_series(x: float, prec: int = 140):
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = prec
        pi = _dec_pi(ctx)
        z = Decimal(repr(x)) / Decimal(2).sqrt()
        term, s, n = z, z, 0
        while True:
            n += 1
            term *= -z * z / n
            d = term / (2 * n + 1)
            s += d
            if n > 10 and abs(d) < Decimal(10) ** (-prec + 5):
                break
        erf = 2 * s / pi.sqrt()
        return Decimal(1) / 2 + erf / 2


def _phi_lower_cf(x: float, depth: int = 4000, prec: int = 60):
    """Phi(-x) for x > 0 by the Mills-ratio continued fraction."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = prec
        pi = _dec_pi(ctx)
        X = Decimal(repr(x))
        r = X
        for k in range(depth, 0, -1):
            r = X + k / r
        dens = (-(X * X) / 2).exp() / (2 * pi).sqrt()
        return dens / r


def test_normal_cdf_references_agree():
    from decimal import Decimal
    for x in (5.0, 6.0, 8.0, 10.0, 12.0):
        a = _phi_series(-x); b = _phi_lower_cf(x)
        assert abs(a - b) <= Decimal(10) ** -35 * b, (x, a, b)
    # textbook anchors: Phi(0) = 1/2, Phi(x) + Phi(-x) = 1
    assert _phi_series(0.0) == Decimal(1) / 2
    assert abs(_phi_series(1.3) + _phi_series(-1.3) - 1) < Decimal(10) ** -100


def test_gelu_textbook_values_and_gradient():
    # the printed table (to the digits it gives), then the series above to
    # near fp64 relative accuracy over the whole range, the far lower tail included
    for x, phi in _read_golden("normal_cdf.txt"):
        x = float(x); phi = float(phi)
        assert abs(O.gelu(np.array([x]))[0] - x * phi) <= 1e-15 * max(abs(x), 1.0)
    # fp64 tolerance from the conditioning of the tail: the argument x / sqrt 2
    # carries a relative rounding error of about 2^-52, and d log Phi / d log x
    # grows like x^2 in the lower tail, so the relative error of Phi(x) computed
    # in fp64 is about (x^2 + 4) 2^-52 (a wrong term or constant is off by far more)
    for x in (-12.0, -10.0, -8.0, -6.5, -5.0, -3.0, -1.0, -0.25, 0.0, 0.25, 1.0, 2.5, 4.0, 8.0):
        ref = float(_phi_series(x))
        got = O.gelu(np.array([x]))[0]
        tol = (x * x + 4.0) * 2.0 ** -52
        assert abs(got - x * ref) <= tol * abs(x * ref), (x, got, x * ref)
    xs = np.linspace(-6, 6, 241)
    h = 1e-6
    fd = (O.gelu(xs + h) - O.gelu(xs - h)) / (2 * h)
    assert np.max(np.abs(fd - O.gelu_grad(xs))) < 1e-8
    # GELU(x) - GELU(-x) = x
    assert np.max(np.abs(O.gelu(xs) - O.gelu(-xs) - xs)) < 1e-14


# ---------------------------------------------------------------- comparison metric
def test_rel_frob_closed_form():
    """||a - b||_F / ||b||_F with b the reference: closed forms that a missing
    square root, a norm of the other argument, or another matrix norm fail."""
    b = np.array([[3.0, 4.0]])                                   # ||b|| = 5
    assert O.rel_frob(np.array([[3.0, 4.5]]), b) == 0.1          # 0.5 / 5 (squared: 0.01)
    assert O.rel_frob(np.array([[6.0, 8.0]]), b) == 1.0          # normalized by ||b||, not ||a|| (0.5)
    assert O.rel_frob(b, np.array([[6.0, 8.0]])) == 0.5
    assert O.rel_frob(np.zeros((1, 2)), b) == 1.0
    # Frobenius, not spectral or max-entry: I + ones vs I gives sqrt(2)
    # (spectral ratio 2, max-entry ratio 1)
    eye = np.eye(2)
    assert abs(O.rel_frob(eye + np.ones((2, 2)), eye) - math.sqrt(2.0)) <= 4.5e-16   # two roundings
    # every element counts, in any layout
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((7, 5)); err = rng.standard_normal((7, 5))
    want = math.sqrt(sum(float(e) ** 2 for e in err.ravel())) / math.sqrt(sum(float(r) ** 2 for r in ref.ravel()))
    assert abs(O.rel_frob(ref + err, ref) - want) <= 1e-14 * want
    assert abs(O.rel_frob((ref + err).T, ref.T) - want) <= 1e-14 * want
    # a zero reference: the absolute norm of the difference
    assert O.rel_frob(b, np.zeros((1, 2))) == 5.0


# ---------------------------------------------------------------- SVD split (Eq. 1)
@pytest.mark.parametrize("shape", [(64, 32, 4), (32, 96, 8)])
def test_svd_split_reconstruction_and_eckart_young(shape):
    N, K, rs = shape
    rng = np.random.default_rng(17)
    spec = synth.LinearSpec("split", 16, K, N, rs, 2, w_outlier_cols=2, w_outlier_mult=20.0)
    d = synth.make_linear(spec, rng)
    W = O.bf16_to_f64(d["W"]); R = O.bf16_to_f64(d["R"])
    L1 = O.bf16_to_f64(d["L1"]); L2 = O.bf16_to_f64(d["L2"])
    chk = O.svd_split_check(W, R, L1, L2)
    # R is W - L1 L2 rounded to bf16: reconstruction within bf16 rounding of R
    assert chk["recon_rel"] < 2 ** -8 * np.linalg.norm(R) / np.linalg.norm(W) + 1e-12
    # Eckart-Young: the rank-rs part leaves the sum of the discarded sigma^2
    # (up to the bf16 rounding of the factors)
    assert abs(chk["resid_sq"] - chk["tail_sq"]) / chk["tail_sq"] < 2e-2
    # an independent decomposition: eigenvalues of W^T W are sigma^2
    ev = np.sort(np.linalg.eigvalsh(W.T @ W))[::-1][:rs]
    assert np.allclose(ev, np.array(chk["top_sv"][:rs]) ** 2, rtol=1e-9)
    # the stabilizer carries the outlier columns: the residual's peak is smaller
    assert np.abs(R).max() < np.abs(W).max()


# --------------------------------------------------------------------------
# pair-merged GEMM operand (a value-preserving re-encoding of Q(x))
# --------------------------------------------------------------------------
def test_e3m2_decode_matches_format_table():
    rows = _read_golden("e3m2_table.txt")
    assert len(rows) == 32
    for code_s, val_s in rows:
        c = int(code_s, 2)
        assert O.e3m2_decode(c) == float(val_s)
        assert O.e3m2_decode(c | 32) == -float(val_s) or float(val_s) == 0.0
    assert np.signbit(O.e3m2_decode(32))


def _operand_case(rng, rows, cols, exps):
    """Random codes with the given scale bytes; a few all-zero blocks."""
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    scales = np.asarray(exps, dtype=np.uint8).reshape(rows // 16, cols // 16)
    zero_blocks = rng.random(scales.shape) < 0.1
    zb = np.repeat(np.repeat(zero_blocks, 16, 0), 16, 1)
    codes = np.where(zb, codes & 8, codes).astype(np.uint8)   # keep signs, zero magnitudes
    return codes, scales


@pytest.mark.parametrize("cols", [16, 48, 112, 128, 144, 400, 528])
def test_operand_decodes_to_the_dequantized_matrix(cols):
    """The operand's values equal Q(x)'s dequantized values, every element, for
    every exponent gap between the blocks of a pair (merged or not), zero
    blocks, the smallest and largest scale bytes, and a ragged last group."""
    rng = np.random.default_rng(cols)
    rows = 64
    nb = (rows // 16) * (cols // 16)
    base = rng.integers(0, 255, size=nb)
    gap = rng.integers(-9, 10, size=nb)
    exps = np.clip(base + gap * (np.arange(nb) % 2), 0, 254)
    exps[:3] = [0, 1, 254]
    codes, scales = _operand_case(rng, rows, cols, exps)
    op, osc = O.operand_merge(codes, scales)
    (r, ob), (sr, sc) = O.operand_shape(rows, cols)
    assert op.shape == (r, ob) and osc.shape == (sr, sc)
    v = O.operand_values(op, osc, rows, cols)
    assert np.array_equal(v[:, :cols], O.dequantize(codes, scales, "pow2"))
    assert np.all(v[:, cols:] == 0)
    # the sign of every element (zeros included) is the sign of its E2M1 code
    sgn = np.signbit(v[:, :cols])
    assert np.array_equal(sgn, (codes >> 3).astype(bool))


def test_operand_merge_rule():
    """Pairs of non-zero blocks merge (equal bytes) exactly when their gap fits the
    E3M2 range: gap <= 5 when the larger byte is >= 2; unmerged pairs keep their
    own bytes."""
    rng = np.random.default_rng(5)
    for e_hi in (0, 1, 2, 7, 127, 254):
        for d in range(0, 9):
            e_lo = e_hi - d
            if e_lo < 0:
                continue
            codes = rng.integers(1, 8, size=(16, 32), dtype=np.uint8)   # no zero blocks
            scales = np.array([[e_hi, e_lo]], np.uint8)
            op, osc = O.operand_merge(codes, scales)
            u = min(d, 2, e_hi)
            if d - u <= 3:
                assert osc[0, 0] == osc[0, 1] == e_hi - u, (e_hi, d)
            else:
                assert (osc[0, 0], osc[0, 1]) == (e_hi, e_lo), (e_hi, d)
            assert np.array_equal(O.operand_values(op, osc, 16, 32)[:, :32],
                                  O.dequantize(codes, scales, "pow2"))
    # a zero block merges with anything, taking the partner's byte
    codes = np.zeros((16, 32), np.uint8)
    codes[:, 16:] = rng.integers(1, 8, size=(16, 16))
    op, osc = O.operand_merge(codes, np.array([[3, 200]], np.uint8))
    assert osc[0, 0] == osc[0, 1] == 200


def test_operand_byte_layout():
    """Hand-built case: positions of single elements in the packed bytes."""
    codes = np.zeros((16, 160), np.uint8)
    codes[0, 0] = 1       # 0.5  -> E3M2 0b01000
    codes[0, 31] = 7      # 6.0  -> E3M2 0b10110
    codes[0, 33] = 10     # -1.0 -> E3M2 0b101100 (sign bit 5)
    codes[0, 128] = 2     # 1.0 in the second group, pair 4
    scales = np.full((1, 10), 127, np.uint8)
    op, osc = O.operand_merge(codes, scales)
    assert op.shape == (16, 192) and osc.shape == (1, 16)
    assert op[0, 0] == 0b01000                        # element 0: bits 0..5 of byte 0
    assert op[0, 64 + 7] == (0b10110 << 2)            # element 31: bits 186..191 = byte 23 (pair 0: slot 0)
    assert op[0, 16] == ((0b101100 << 6) & 0xFF)      # pair 1, element 1: bits 6..11
    assert op[0, 17] == (0b101100 >> 2)
    assert op[0, 96] == 0b01100                       # pair 4 = group 1, first chunk
    assert np.count_nonzero(op) == 4                  # byte 16 holds only zero bits of it
    # pair 1's last 8 bytes sit in slot 2 (order 0, 2, 1, 3): element 31 of pair 1
    c3 = np.zeros((16, 128), np.uint8)
    c3[0, 63] = 7
    op3, _ = O.operand_merge(c3, np.full((1, 8), 127, np.uint8))
    assert op3[0, 64 + 16 + 7] == (0b10110 << 2) and np.count_nonzero(op3) == 1
    assert np.all(osc[0, :10] == 127) and np.all(osc[0, 10:] == 0)
    # shift: block bytes 127 and 125 (gap 2) merge at 125; the first block's values x4
    codes2 = np.zeros((16, 32), np.uint8)
    codes2[0, 0] = 7      # 6.0 * 2^0 -> shifted to 24.0 = E3M2 0b11110
    codes2[0, 16] = 1     # 0.5 in the second block, unshifted
    op2, osc2 = O.operand_merge(codes2, np.array([[127, 125]], np.uint8))
    assert osc2[0, 0] == osc2[0, 1] == 125
    assert op2[0, 0] == 0b11110
    assert (int.from_bytes(bytes(op2[0, :16]), "little") >> 96) & 63 == 0b01000


def test_operand_of_the_transpose():
    """The operand of Q(x)^T (codes and scale grid transposed) decodes to the transposed values."""
    rng = np.random.default_rng(8)
    x = synth.f32_to_bf16_bits(synth.make_tensor(rng, (96, 160), "t3"))
    codes, scales = O.quantize_block16(x)
    op, osc = O.operand_merge(codes.T, scales.T)
    v = O.operand_values(op, osc, 160, 96)
    assert np.array_equal(v[:, :96], O.dequantize(codes, scales, "pow2").T)


# ---------------------------------------------------------------- group granularities
@pytest.mark.parametrize("g", [16, 32])
def test_group_quantizer_elementwise_bruteforce(g):
    """1 x g groups along each row: scale byte and every code re-derived by
    exact rational brute force (section 4.3, Table 5's group-wise setting)."""
    rng = np.random.default_rng(17 + g)
    x = (rng.standard_normal((6, 96)) * np.exp2(rng.integers(-6, 6, (6, 96)))).astype(np.float32)
    x[2, :g] = 0.0
    x[3, g:2 * g] = -0.0
    bits = synth.f32_to_bf16_bits(x)
    codes, scales = O.quantize_groups(bits, g)
    assert codes.shape == (6, 96) and scales.shape == (6, 96 // g)
    xv = O.bf16_to_f64(bits)
    for i in range(6):
        for q in range(96 // g):
            grp = xv[i, g * q:g * q + g]
            E = _pow2_bruteforce(Fraction(float(np.abs(grp).max())))
            assert scales[i, q] == E + 127
            for j in range(g):
                v = float(grp[j])
                ratio = float(Fraction(v) / Fraction(2) ** E) if v != 0 else v
                assert codes[i, g * q + j] == _rne_bruteforce(ratio), (i, q, j)


def test_group_quantizer_reduces_to_16x16_blocks():
    """When every row of a 16x16 block reaches the block's maximum, the 1 x 16
    groups and the 16 x 16 blocks take the same scale and the same codes."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    xv = O.bf16_to_f64(bits).astype(np.float32)
    for bi in range(2):
        for bj in range(4):
            blk = xv[16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16]
            m = np.abs(blk).max()
            for r in range(16):
                blk[r, (r * 5) % 16] = m if r % 2 else -m
    bits = synth.f32_to_bf16_bits(xv)
    cg, sg = O.quantize_groups(bits, 16)
    cb, sb = O.quantize_block16(bits, "pow2")
    assert np.array_equal(cg, cb)
    assert np.array_equal(sg, np.repeat(sb, 16, axis=0))


def _dequant_group_exact(codes, scales, g):
    """Exact rational values of a group-quantized matrix from the code table."""
    vals = {}
    for bits, val in _read_golden("e2m1_table.txt"):
        vals[int(bits, 2)] = Fraction(float(val))
    rows, cols = codes.shape
    return [[vals[int(codes[i, j])] * Fraction(2) ** (int(scales[i, j // g]) - 127) for j in range(cols)]
            for i in range(rows)]


@pytest.mark.parametrize("g", [16, 32])
def test_requantize_transposed_bruteforce(g):
    """Q_g(deq(Q_g(R))^T): the transpose of the exact dequantized values,
    quantized again by brute force in groups along R's columns."""
    rng = np.random.default_rng(31 + g)
    R = (rng.standard_normal((2 * g, 64)) * np.exp2(rng.integers(-5, 5, (2 * g, 64)))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(R)
    c, s = O.quantize_groups(bits, g)
    ct, st = O.requantize_transposed(c, s, g)
    assert ct.shape == (64, 2 * g) and st.shape == (64, 2)
    D = _dequant_group_exact(c, s, g)
    for col in range(64):
        for q in range(2):
            grp = [D[g * q + r][col] for r in range(g)]
            E = _pow2_bruteforce(max(abs(v) for v in grp))
            assert st[col, q] == E + 127
            for r in range(g):
                v = grp[r]
                code = int(c[g * q + r, col])
                ratio = float(v / Fraction(2) ** E)
                if v == 0:   # a zero keeps the sign bit of its code
                    assert ct[col, g * q + r] == (code & 8)
                else:
                    assert ct[col, g * q + r] == _rne_bruteforce(ratio)


def test_requantize_transposed_lossless_when_groups_share_the_maximum():
    """If every group along the rows and along the columns holds a +-6 x 2^E
    element (one common E) and all values are E2M1 values x 2^E, quantizing,
    transposing and quantizing again loses nothing: the codes are transposed."""
    rng = np.random.default_rng(41)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    v = grid[rng.integers(0, 8, (32, 64))] * rng.choice([-1.0, 1.0], (32, 64))
    for i in range(32):
        for j in range(4):
            v[i, 16 * j + (i % 16)] = 6.0 if (i + j) % 2 else -6.0
    v *= 2.0 ** -3
    bits = synth.f32_to_bf16_bits(v.astype(np.float32))
    c, s = O.quantize_groups(bits, 16)
    assert np.all(s == 127 - 3)
    ct, st = O.requantize_transposed(c, s, 16)
    assert np.all(st == 127 - 3)
    nz = (c.T & 7) != 0
    assert np.array_equal(ct[nz], c.T[nz])
    assert np.array_equal(O.dequantize_pow2(ct, st, 1, 16), O.bf16_to_f64(bits).T)


def test_rel_mse_closed_form():
    x = np.array([[3.0, 4.0]])
    assert O.rel_mse(x, np.array([[3.0, 0.0]])) == 16.0 / 25.0
    assert O.rel_mse(x, x) == 0.0
