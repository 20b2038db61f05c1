"""Plain fp64 CPU oracle of the FourTune W4A4G4 triple-branch linear.

Test infrastructure only (see the package docstring).  Conventions:

* bf16 tensors arrive as uint16 bit patterns (``bits``) and are decoded
  exactly to float64.
* A quantized matrix is described by its unpacked 4-bit codes ``codes``
  (uint8 in 0..15, same shape as the input) and its scale grid
  ``scales`` of shape [rows/16, cols/16].
* Scale rules (the pages fix "scale from the block maximum" but not its
  number format; both readings are implemented):
    - "f32":  s = fl32(amax / 6), IEEE binary32 division (round to nearest
      even); the element ratio is v = fl32(x / s).
    - "pow2": s = 2^E with E the smallest integer such that 6 * 2^E >= amax,
      clamped to [-127, 127] (the E8M0 scale byte is E + 127); the element
      ratio is v = x * 2^-E, exact.  This is amax / 6 rounded up to a power
      of two, so no element saturates.
  A block whose maximum is zero gets s = 0 ("f32") or byte 0 ("pow2") and
  all-zero codes.
* E2M1 code = sign << 3 | exponent(2 bits, bias 1) << 1 | mantissa(1 bit);
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Rounding is to the nearest
  magnitude, ties to the code with mantissa bit 0, |v| > 6 saturates to 6,
  and the sign bit is the sign bit of the input (so -0 gives code 8).
* Packing: two codes per byte, the element with the even index in the low
  nibble.  Row-major: element (i, j) in byte (i*cols + j) // 2.
  Column-major: element (i, j) in byte (j*rows + i) // 2.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16_bits", "e2m1_decode", "e2m1_rne",
    "block_amax", "scale_pow2_exponent", "scale_f32", "quantize_block16",
    "pack_rm", "pack_cm", "unpack_rm", "dequantize", "scale_values",
    "linear_fwd", "linear_bwd", "gelu", "gelu_grad", "svd_split_check",
    "rel_frob", "BLOCK", "quantize_pow2", "dequantize_pow2", "quantize_groups",
    "requantize_transposed", "rel_mse",
    "e3m2_decode", "OP_GROUP", "operand_merge", "operand_values", "operand_shape",
]

BLOCK = 16


# --------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of binary32)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 with round-to-nearest-even (finite inputs).

    Written as an explicit nearest-neighbour choice between the two bf16
    values that bracket x: the truncation t (x rounded toward zero to 8
    significant bits) and the next value away from zero; the tie goes to
    the one whose last mantissa bit is 0.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(np.abs(x))              # |x| = m * 2^e, m in [0.5, 1)
    # bf16 keeps 8 significant bits for normal numbers (2^-126 and up) and
    # a fixed quantum of 2^-133 below that.
    q_exp = np.maximum(e - 8, -133)          # quantum (last-bit weight) exponent
    q = np.ldexp(1.0, q_exp)
    n = np.abs(x) / q                        # exact: power-of-two division
    lo = np.floor(n)
    frac = n - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.fmod(lo, 2) == 1))
    mag = (lo + up) * q
    y = np.where(np.signbit(x), -mag, mag).astype(np.float32)
    return (y.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------
def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes from the format definition.

    exponent field e (2 bits, bias 1), mantissa bit m:
      e == 0: subnormal, magnitude m * 0.5
      e >= 1: magnitude (1 + m/2) * 2^(e-1)
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(sign == 1, -mag, mag)


# magnitude thresholds of round-to-nearest-even on the E2M1 grid
# 0 | 0.5 | 1 | 1.5 | 2 | 3 | 4 | 6 : a value moves to the next magnitude
# when it passes the midpoint; on the midpoint it moves only if the next
# code has mantissa bit 0 (codes 2, 4, 6), i.e. at 0.75, 1.75 and 3.5.
_MID = [(0.25, False), (0.75, True), (1.25, False), (1.75, True),
        (2.5, False), (3.5, True), (5.0, False)]


def e2m1_rne(v) -> np.ndarray:
    """Round fp64 ratios to E2M1 codes: nearest, ties to even, saturate at 6.

    The sign bit of the code is the sign bit of ``v`` (-0 -> code 8).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    mag_code = np.zeros(v.shape, dtype=np.uint8)
    for mid, inclusive in _MID:
        mag_code += (a >= mid if inclusive else a > mid).astype(np.uint8)
    return (np.signbit(v).astype(np.uint8) << 3) | mag_code


# --------------------------------------------------------------------------
# 16x16 block quantizer (sections 3.1 and 3.2)
# --------------------------------------------------------------------------
def _blocks(x: np.ndarray) -> np.ndarray:
    r, c = x.shape
    assert r % BLOCK == 0 and c % BLOCK == 0, "rows and cols must be multiples of 16"
    return x.reshape(r // BLOCK, BLOCK, c // BLOCK, BLOCK)


def block_amax(x: np.ndarray) -> np.ndarray:
    """max |x| over each 16x16 block -> [rows/16, cols/16]."""
    return np.abs(_blocks(x)).max(axis=(1, 3))


def scale_pow2_exponent(amax) -> np.ndarray:
    """E = min{e integer : 6 * 2^e >= amax}, clamped to [-127, 127] (E = -127 for amax 0).

    6 * 2^e >= amax  <=>  e >= log2(amax / 6).  frexp gives amax/6 = f * 2^p
    with f in [0.5, 1); the smallest such e is p - 1 when f == 0.5 (amax/6 a
    power of two) and p otherwise.  amax/6 is computed in fp64; amax has at
    most 8 significant bits, so the quotient is a power of two only when it
    is exactly one.
    """
    a = np.asarray(amax, dtype=np.float64)
    f, p = np.frexp(a / 6.0)
    e = np.where(f == 0.5, p - 1, p).astype(np.int64)
    e = np.where(a == 0.0, -127, e)
    return np.clip(e, -127, 127)


def scale_f32(amax) -> np.ndarray:
    """s = fl32(amax / 6), IEEE binary32 division."""
    a = np.asarray(amax, dtype=np.float64).astype(np.float32)
    with np.errstate(all="ignore"):
        return (a / np.float32(6.0)).astype(np.float32)


def quantize_block16(bits, mode: str = "pow2") -> Tuple[np.ndarray, np.ndarray]:
    """Q(.) of a bf16 matrix: unpacked codes [rows, cols] and the scale grid.

    Returns (codes uint8, scales) where scales is uint8 E8M0 bytes
    (mode "pow2") or float32 (mode "f32"), shape [rows/16, cols/16].
    """
    x = bf16_to_f64(bits)
    rows, cols = x.shape
    amax = block_amax(x)
    xb = _blocks(x)
    if mode == "pow2":
        E = scale_pow2_exponent(amax)
        v = xb * np.exp2(-E.astype(np.float64))[:, None, :, None]   # exact
        scales = (E + 127).astype(np.uint8)
    elif mode == "f32":
        s = scale_f32(amax)
        x32 = xb.astype(np.float32)                                  # exact (bf16 subset of f32)
        with np.errstate(all="ignore"):
            v32 = x32 / s[:, None, :, None]                          # IEEE binary32 division
        # a block with amax == 0 has s == 0 and only (+-)0 elements: ratio (+-)0
        zero_blk = (s == 0)[:, None, :, None] & np.ones_like(v32, dtype=bool)
        v32 = np.where(zero_blk, x32 * np.float32(0.0), v32)
        v = v32.astype(np.float64)
        scales = s
    else:
        raise ValueError(mode)
    codes = e2m1_rne(v).reshape(rows, cols)
    return codes, scales


def scale_values(scales, mode: str) -> np.ndarray:
    """fp64 value of each block scale."""
    if mode == "pow2":
        return np.exp2(np.asarray(scales).astype(np.float64) - 127.0)
    return np.asarray(scales, dtype=np.float32).astype(np.float64)


def dequantize(codes, scales, mode: str) -> np.ndarray:
    """Exact fp64 value of a block-quantized matrix: code value * block scale."""
    vals = e2m1_decode(codes)
    s = scale_values(scales, mode)
    return vals * np.repeat(np.repeat(s, BLOCK, 0), BLOCK, 1)


def pack_rm(codes) -> np.ndarray:
    """Row-major packing: [rows, cols/2], even column in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_rm(packed, cols: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], cols), np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def pack_cm(codes) -> np.ndarray:
    """Column-major packing: [cols, rows/2]; byte (j, i/2) holds rows i, i+1 of column j."""
    return pack_rm(np.asarray(codes, dtype=np.uint8).T)


# --------------------------------------------------------------------------
# GEMM operand: the same Q(x), re-encoded with pairs of blocks merged
# --------------------------------------------------------------------------
# Not a step of the method: a value-preserving re-encoding of a quantized
# matrix (pow2 scales) in which the two 16-column blocks of each 32-column
# pair share one power-of-two scale, so that one 32-value, one-scale fragment
# of a block-scaled matrix instruction carries both blocks.  Its only
# contract is operand_values(operand_merge(codes, scales)) == dequantize(codes,
# scales) exactly.  Elements are FP6 E3M2 (OCP Microscaling Formats v1.0,
# section 5.3.2: 1 sign, 3 exponent bits with bias 3, 2 mantissa bits, no
# Inf/NaN; magnitudes 0.0625 .. 28).
#
# Encoding of one pair (row block rb, blocks b1 = 2p, b2 = 2p + 1), with the
# E8M0 bytes e1, e2 of the blocks:
#  * a block whose codes are all +-0 takes its partner's byte (its scale does
#    not matter); if both are, both take max(e1, e2);
#  * d = |e1 - e2|, hi = max(e1, e2), u = min(d, 2, hi).  The pair is merged
#    when d - u <= 3: both blocks then use the byte H = hi - u, and an element
#    of block b becomes the E3M2 value e2m1(code) * 2^(e_b - H), a shift of
#    +u for the larger block and u - d >= -3 for the other, always exact;
#  * otherwise (d - u > 3) each block keeps its own byte and its values are
#    the E2M1 values (shift 0).  Merged pairs have equal bytes, unmerged
#    pairs different ones, which is how a consumer tells them apart.
#  The sign bit of every element is the sign bit of its E2M1 code.
#
# Layout: the column index is padded to a multiple of OP_GROUP = 128 (4 pairs;
# padding is all-zero codes with scale byte 0).  A row of the operand has
# 96 bytes per group: the first 16 bytes of the 24-byte packed value of pairs
# 0..3 of the group (64 bytes), then the last 8 bytes of pairs 0, 2, 1, 3 in
# that order (32 bytes: a 16-byte unit per pair parity).  The
# 24-byte value of a pair holds its 32 elements, element n (column 32p + n)
# in bits 6n .. 6n+5, little-endian.  The scale grid is [rows/16, 8 * groups]
# bytes: entries 2p and 2p + 1 of row block rb are the bytes of blocks b1, b2.
OP_GROUP = 128
_HPOS = (0, 2, 1, 3)   # slot of pair q's last 8 bytes among the group's four


def e3m2_decode(codes) -> np.ndarray:
    """Value of 6-bit E3M2 codes from the format definition.

    exponent field e (3 bits, bias 3), mantissa m (2 bits):
      e == 0: subnormal, magnitude (m / 4) * 2^-2
      e >= 1: magnitude (1 + m/4) * 2^(e-3)
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 5) & 1
    e = (c >> 2) & 7
    m = c & 3
    mag = np.where(e == 0, (m / 4.0) * 0.25, (1.0 + m / 4.0) * np.exp2(e - 3.0))
    return np.where(sign == 1, -mag, mag)


def _e3m2_code_of(mag) -> np.ndarray:
    """The E3M2 magnitude code (0..31) whose value equals ``mag`` exactly."""
    table = e3m2_decode(np.arange(32))
    mag = np.asarray(mag, dtype=np.float64)
    idx = np.searchsorted(table, mag)
    idx = np.minimum(idx, 31)
    if not np.all(table[idx] == mag):
        raise ValueError("value not representable in E3M2")
    return idx.astype(np.uint8)


def operand_shape(rows: int, cols: int) -> Tuple[Tuple[int, int], Tuple[int, int]]:
    """(operand bytes shape, operand scale grid shape) of a [rows, cols] matrix."""
    g = -(-cols // OP_GROUP)
    return (rows, 96 * g), (rows // BLOCK, 8 * g)


def operand_merge(codes, scales) -> Tuple[np.ndarray, np.ndarray]:
    """Pair-merged operand of a pow2-quantized matrix (codes [rows, cols], bytes)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows, cols = codes.shape
    (_, obytes), (srows, scols) = operand_shape(rows, cols)
    g = obytes // 96
    P = 4 * g                                      # pairs per row (with padding)
    cpad = np.zeros((rows, 32 * P), np.uint8)
    cpad[:, :cols] = codes
    epad = np.zeros((rows // BLOCK, 2 * P), np.int64)
    epad[:, :cols // BLOCK] = scales
    # zero blocks: every code of the block has magnitude 0
    mag_blk = (cpad & 7).reshape(rows // BLOCK, BLOCK, 2 * P, BLOCK)
    zero = ~mag_blk.any(axis=(1, 3))               # [rows/16, 2P]
    e1, e2 = epad[:, 0::2], epad[:, 1::2]
    z1, z2 = zero[:, 0::2], zero[:, 1::2]
    both = z1 & z2
    f1 = np.where(both, np.maximum(e1, e2), np.where(z1, e2, e1))
    f2 = np.where(both, np.maximum(e1, e2), np.where(z2, e1, e2))
    d = np.abs(f1 - f2)
    hi = np.maximum(f1, f2)
    u = np.minimum(np.minimum(d, 2), hi)
    merged = (d - u) <= 3
    H = hi - u
    s1 = np.where(merged, H, e1)
    s2 = np.where(merged, H, e2)
    t1 = np.where(merged, f1 - H, 0)               # exponent shift of each block's values
    t2 = np.where(merged, f2 - H, 0)
    # element shifts [rows, 32P]
    t = np.stack([t1, t2], axis=-1).reshape(rows // BLOCK, 2 * P)
    t_el = np.repeat(np.repeat(t, BLOCK, axis=0), BLOCK, axis=1)
    vals = np.abs(e2m1_decode(cpad)) * np.exp2(t_el.astype(np.float64))
    c6 = _e3m2_code_of(vals) | ((cpad >> 3) << 5)
    # pack 32 six-bit codes per pair into 24 little-endian bytes
    c6 = c6.reshape(rows, P, 32)
    bits = ((c6[..., None] >> np.arange(6, dtype=np.uint8)) & 1).reshape(rows, P, 192)
    packed = np.packbits(bits, axis=-1, bitorder="little")          # [rows, P, 24]
    op = np.zeros((rows, obytes), np.uint8)
    for p in range(P):
        grp, q = divmod(p, 4)
        op[:, 96 * grp + 16 * q: 96 * grp + 16 * q + 16] = packed[:, p, :16]
        h = 64 + 8 * _HPOS[q]
        op[:, 96 * grp + h: 96 * grp + h + 8] = packed[:, p, 16:]
    osc = np.zeros((srows, scols), np.uint8)
    osc[:, 0::2] = s1
    osc[:, 1::2] = s2
    return op, osc


def operand_values(op, op_scales, rows: int, cols: int) -> np.ndarray:
    """fp64 values [rows, 128 * groups] encoded by an operand (padding included)."""
    op = np.asarray(op, dtype=np.uint8)
    g = op.shape[1] // 96
    P = 4 * g
    packed = np.empty((rows, P, 24), np.uint8)
    for p in range(P):
        grp, q = divmod(p, 4)
        packed[:, p, :16] = op[:, 96 * grp + 16 * q: 96 * grp + 16 * q + 16]
        h = 64 + 8 * _HPOS[q]
        packed[:, p, 16:] = op[:, 96 * grp + h: 96 * grp + h + 8]
    bits = np.unpackbits(packed, axis=-1, bitorder="little").reshape(rows, P, 32, 6)
    c6 = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)      # [rows, P, 32]
    v = e3m2_decode(c6).reshape(rows, 32 * P)
    s = np.exp2(np.asarray(op_scales).astype(np.float64) - 127.0)  # [rows/16, 2P]
    return v * np.repeat(np.repeat(s, BLOCK, 0), BLOCK, 1)


# --------------------------------------------------------------------------
# Other quantization granularities (section 4.3 "Impact of Quantization
# Granularity", Table 5: group-wise 1x16 against the 16x16 blocks; section
# 3.2: group scales along a row end up along the reduction axis of the
# transposed product)
# --------------------------------------------------------------------------
# Reading: a 1 x g group is g consecutive elements of one row (the reduction
# axis of the forward product), with the same element rule (E2M1,
# round-to-nearest-even, sign of the input) and the same pow2 scale rule as the
# 16x16 blocks.  g = 16 is the paper's group-wise setting; g = 32 is the group
# length the gfx950 block-scaled matrix instruction takes per scale.  The
# transposed product of the backward reduces over R's rows, across R's groups,
# so with group scales Q(R) is dequantized and quantized again in groups along
# its columns: Q_g(deq(Q_g(R))^T).
def quantize_pow2(x, bh: int, bw: int) -> Tuple[np.ndarray, np.ndarray]:
    """pow2-rule Q(.) of an fp64 matrix over bh x bw blocks.

    Returns (codes uint8 [rows, cols], scale bytes uint8 [rows/bh, cols/bw]);
    E per block from the block maximum (scale_pow2_exponent), element ratio
    x * 2^-E (exact), E2M1 round-to-nearest-even (e2m1_rne).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % bh == 0 and cols % bw == 0, "shape must be a multiple of the block"
    xb = x.reshape(rows // bh, bh, cols // bw, bw)
    E = scale_pow2_exponent(np.abs(xb).max(axis=(1, 3)))
    v = xb * np.exp2(-E.astype(np.float64))[:, None, :, None]
    return e2m1_rne(v).reshape(rows, cols), (E + 127).astype(np.uint8)


def dequantize_pow2(codes, scales, bh: int, bw: int) -> np.ndarray:
    """Exact fp64 value of a pow2-quantized matrix with bh x bw blocks."""
    s = np.exp2(np.asarray(scales).astype(np.float64) - 127.0)
    return e2m1_decode(codes) * np.repeat(np.repeat(s, bh, 0), bw, 1)


def quantize_groups(bits, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """Q(.) of a bf16 matrix in 1 x g groups along its rows: codes [rows, cols]
    and scale bytes [rows, cols/g]."""
    return quantize_pow2(bf16_to_f64(bits), 1, g)


def requantize_transposed(codes, scales, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """The backward's right operand under 1 x g groups: the values of Q_g(R)
    transposed and quantized again in 1 x g groups, Q_g(deq(Q_g(R))^T).
    codes [rows, cols], scales [rows, cols/g] of R -> codes [cols, rows],
    scales [cols, rows/g]."""
    return quantize_pow2(dequantize_pow2(codes, scales, 1, g).T, 1, g)


def rel_mse(x, xhat) -> float:
    """||x - xhat||^2 / ||x||^2 in fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x - np.asarray(xhat, dtype=np.float64)
    n = float(np.sum(x * x))
    return float(np.sum(d * d)) / n if n > 0 else 0.0


# --------------------------------------------------------------------------
# Triple-branch linear (Eq. 2, Eq. 3, adapter gradients)
# --------------------------------------------------------------------------
def linear_fwd(Xhat, Rhat, X, L1, L2, A, B) -> np.ndarray:
    """Eq. 2: Y = Q(X) Q(R)^T + X (L1 L2) + X (A B).

    Xhat [M,K] and Rhat [N,K] are the dequantized Q(X), Q(R) (R in out x in
    layout, so the backbone term is Xhat Rhat^T); X is the unquantized
    input; L1 [K,rs], L2 [rs,N], A [K,r], B [r,N].  All fp64.
    """
    backbone = Xhat @ Rhat.T
    stabilizer = X @ (L1 @ L2)
    adapter = X @ (A @ B)
    return backbone + stabilizer + adapter


def linear_bwd(Ghat, Rhat, G, X, L1, L2, A, B) -> Dict[str, np.ndarray]:
    """Eq. 3 and the adapter gradients of section 3.2.

    dX = Q(G) Q(R) + G (L1 L2)^T + G (A B)^T   (Q(R) in out x in layout,
         so GEMM_4bit(Q(G), Q(R)^T) of the paper's in x out layout is Ghat Rhat)
    dB = (X A)^T G,   dA = X^T (G B^T).
    Q is treated as the identity when differentiating (no gradient flows to
    R, L1 or L2).
    """
    dX = Ghat @ Rhat + G @ (L1 @ L2).T + G @ (A @ B).T
    dB = (X @ A).T @ G
    dA = X.T @ (G @ B.T)
    return {"dX": dX, "dA": dA, "dB": dB}


def _norm_cdf(x) -> np.ndarray:
    """Standard normal CDF Phi(x) = erfc(-x / sqrt(2)) / 2.

    The complementary-error-function form keeps full relative accuracy in the
    lower tail, where 1 + erf(x / sqrt 2) cancels to zero (x below about -8).
    """
    from scipy.special import erfc
    return 0.5 * erfc(-np.asarray(x, dtype=np.float64) / math.sqrt(2.0))


def gelu(x) -> np.ndarray:
    """GELU(x) = x * Phi(x), Phi the standard normal CDF."""
    x = np.asarray(x, dtype=np.float64)
    return x * _norm_cdf(x)


def gelu_grad(x) -> np.ndarray:
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    x = np.asarray(x, dtype=np.float64)
    phi = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return _norm_cdf(x) + x * phi


def svd_split_check(W, R, L1, L2) -> Dict[str, float]:
    """Checks of the offline split W ~= R + L1 L2 (Eq. 1) in fp64.

    W, R in out x in layout [N,K]; L1 [K,rs], L2 [rs,N].  Returns the
    relative reconstruction error of R + (L1 L2)^T and the Eckart-Young gap:
    ||W - (L1 L2)^T||_F^2 compared with the sum of the discarded squared
    singular values of W.
    """
    W = np.asarray(W, np.float64); R = np.asarray(R, np.float64)
    Ls = (np.asarray(L1, np.float64) @ np.asarray(L2, np.float64)).T
    rs = np.asarray(L1).shape[1]
    sv = np.linalg.svd(W, compute_uv=False)
    tail = float(np.sum(sv[rs:] ** 2))
    resid = float(np.sum((W - Ls) ** 2))
    return {
        "recon_rel": float(np.linalg.norm(R + Ls - W) / np.linalg.norm(W)),
        "resid_sq": resid,
        "tail_sq": tail,
        "top_sv": sv[: max(rs, 1)].tolist(),
    }


def rel_frob(a, b) -> float:
    """||a - b||_F / ||b||_F (b is the reference)."""
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))
