"""Seeded synthetic inputs for the W4A4G4 triple-branch linear.

This module is shared by the CPU oracle (``oracle/``) and by the GPU path's
tests and benchmark.  It draws random tensors and rounds them to bf16; it
holds none of the quantization or GEMM arithmetic of the method.

The one preparation step it performs is the offline stabilizer split of the
frozen weight (FourTune, "3.1 Triple-Branch Hybrid-Precision Pipeline",
Eq. 1: W ~= R + L1 L2 with L1 L2 a truncated SVD).  The split is not unique
(singular-vector signs, how the singular values are shared between L1 and
L2), so it is computed once here and the same factors are handed to both
sides; the oracle pins it independently (reconstruction, Eckart-Young).

Shapes follow the layer convention used across the project:
  X  [M x K]  activations (tokens x in-features), bf16
  W  [N x K]  frozen weight (out x in), bf16
  R  [N x K]  residual after the split, bf16
  L1 [K x rs], L2 [rs x N]  stabilizer factors (paper layout, Y = X W^T = X Wp)
  A  [K x r],  B  [r x N]   LoRA factors
  G  [M x N]  incoming gradient dL/dY, bf16

bf16 tensors are carried as numpy uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "LinearSpec", "CONFIGS",
    "make_linear", "make_tensor", "edge_tensor", "config_linears",
]


# --------------------------------------------------------------------------
# bf16 helpers (input synthesis only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), return uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Config recipes (FLUX.1-dev shaped linears: hidden 3072, MLP 12288,
# 4096 image + 512 text tokens at 1024^2).
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LinearSpec:
    name: str
    M: int
    K: int
    N: int
    rs: int          # stabilizer rank
    r: int           # LoRA rank
    x_dist: str = "normal"      # "normal" | "t3"
    x_outlier_frac: float = 0.0  # fraction of input channels scaled
    x_outlier_count: int = 0     # or an explicit count
    x_outlier_mult: float = 1.0
    w_std: float = 0.02
    w_outlier_cols: int = 0
    w_outlier_mult: float = 1.0
    a_std: float = 0.01
    b_mult: float = 0.01
    g_std: float = 1e-3

    @property
    def rho(self) -> int:
        return self.rs + self.r


def _c5_specs() -> List[LinearSpec]:
    out = []
    for stream, M in (("img", 4096), ("txt", 512)):
        out += [
            LinearSpec(f"c5-{stream}-qkv", M, 3072, 9216, 32, 32),
            LinearSpec(f"c5-{stream}-proj", M, 3072, 3072, 32, 32),
            LinearSpec(f"c5-{stream}-up", M, 3072, 12288, 32, 32),
            LinearSpec(f"c5-{stream}-down", M, 12288, 3072, 32, 32),
        ]
    return out


CONFIGS: Dict[str, List[LinearSpec]] = {
    # single linear 256^3: 4 outlier activation channels x30, 2 outlier weight input columns x20
    "c1": [LinearSpec("c1", 256, 256, 256, 16, 16, x_outlier_count=4, x_outlier_mult=30.0,
                      w_outlier_cols=2, w_outlier_mult=20.0)],
    # attention projection: 1% channels x50
    "c2": [LinearSpec("c2", 4608, 3072, 3072, 32, 32, x_outlier_frac=0.01, x_outlier_mult=50.0)],
    # MLP pair with Student-t(3) activations; GELU between the two linears
    "c3": [LinearSpec("c3-up", 4608, 3072, 12288, 32, 16, x_dist="t3"),
           LinearSpec("c3-down", 4608, 12288, 3072, 32, 16, x_dist="t3")],
    # fused QKV at batch 4: 0.5% channels x100
    "c4": [LinearSpec("c4", 18432, 3072, 9216, 64, 64, x_outlier_frac=0.005, x_outlier_mult=100.0)],
    # double-stream block linear stack
    "c5": _c5_specs(),
}

CONFIG_SEED = {"c1": 1000, "c2": 1001, "c3": 1002, "c4": 1003, "c5": 1004}


def _outlier_count(spec: LinearSpec) -> int:
    if spec.x_outlier_count:
        return spec.x_outlier_count
    return int(round(spec.x_outlier_frac * spec.K))


def make_tensor(rng: np.random.Generator, shape, dist: str = "normal", std: float = 1.0) -> np.ndarray:
    """Draw a float32 tensor with the given distribution (std is the standard deviation)."""
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
    elif dist == "t3":
        x = rng.standard_t(3, size=shape).astype(np.float32)
        if std != 1.0:
            x *= np.float32(std)
    else:
        raise ValueError(dist)
    return x


def _split(W_bits: np.ndarray, rs: int):
    """Offline stabilizer split of a frozen weight (Eq. 1), computed once.

    W is [N x K] (out x in).  The paper's weight is Wp = W^T [K x N] with
    Y = X Wp.  L1 L2 is the rank-rs truncated SVD of Wp with the singular
    values shared as sqrt between the factors; the factors are rounded to
    bf16 and the residual R = W - (L1 L2)^T is formed in fp64 from the
    rounded factors and rounded to bf16.
    """
    Wp = bf16_bits_to_f32(W_bits).astype(np.float64).T  # [K x N]
    K, N = Wp.shape
    if rs == 0:
        L1 = np.zeros((K, 0)); L2 = np.zeros((0, N))
    elif K <= N:
        C = Wp @ Wp.T
        w, P = np.linalg.eigh(C)
        idx = np.argsort(w)[::-1][:rs]
        sig = np.sqrt(np.maximum(w[idx], 0.0))
        Pr = P[:, idx]
        L1 = Pr * np.sqrt(sig)[None, :]
        L2 = (Pr.T @ Wp) / np.sqrt(sig)[:, None]
    else:
        C = Wp.T @ Wp
        w, Q = np.linalg.eigh(C)
        idx = np.argsort(w)[::-1][:rs]
        sig = np.sqrt(np.maximum(w[idx], 0.0))
        Qr = Q[:, idx]
        L2 = (Qr * np.sqrt(sig)[None, :]).T
        L1 = (Wp @ Qr) / np.sqrt(sig)[None, :]
    L1b = f32_to_bf16_bits(L1.astype(np.float32))
    L2b = f32_to_bf16_bits(L2.astype(np.float32))
    L1r = bf16_bits_to_f32(L1b).astype(np.float64)
    L2r = bf16_bits_to_f32(L2b).astype(np.float64)
    Rp = Wp - L1r @ L2r
    R = f32_to_bf16_bits(np.ascontiguousarray(Rp.T).astype(np.float32))
    return R, L1b, L2b


def make_linear(spec: LinearSpec, rng: np.random.Generator, with_x: bool = True,
                with_g: bool = True) -> Dict[str, np.ndarray]:
    """Draw one linear's inputs: outlier indices, X, W, A, B, G in that order."""
    out: Dict[str, np.ndarray] = {}
    nout = _outlier_count(spec)
    x_cols = rng.choice(spec.K, size=nout, replace=False) if nout else np.zeros(0, np.int64)
    w_cols = (rng.choice(spec.K, size=spec.w_outlier_cols, replace=False)
              if spec.w_outlier_cols else np.zeros(0, np.int64))
    out["x_outlier_cols"] = np.sort(x_cols)
    if with_x:
        X = make_tensor(rng, (spec.M, spec.K), spec.x_dist)
        if nout:
            X[:, x_cols] *= np.float32(spec.x_outlier_mult)
        out["X"] = f32_to_bf16_bits(X)
    W = make_tensor(rng, (spec.N, spec.K), "normal", spec.w_std)
    if spec.w_outlier_cols:
        W[:, w_cols] *= np.float32(spec.w_outlier_mult)
    out["W"] = f32_to_bf16_bits(W)
    out["A"] = f32_to_bf16_bits(make_tensor(rng, (spec.K, spec.r), "normal", spec.a_std))
    out["B"] = f32_to_bf16_bits(make_tensor(rng, (spec.r, spec.N), "normal", 1.0) * np.float32(spec.b_mult))
    if with_g:
        out["G"] = f32_to_bf16_bits(make_tensor(rng, (spec.M, spec.N), "normal", spec.g_std))
    R, L1, L2 = _split(out["W"], spec.rs)
    out["R"], out["L1"], out["L2"] = R, L1, L2
    return out


def config_linears(cfg: str, scale_m: Optional[int] = None) -> List[Dict[str, np.ndarray]]:
    """All linears of a config, drawn from the config's seed in stack order.

    ``scale_m`` replaces M (tokens) when a smaller case of the same recipe is
    wanted.  For chained stacks the X of the second linear of a pair is not
    drawn (it is the GELU of the first linear's output); every linear draws
    its own G.
    """
    rng = np.random.default_rng(CONFIG_SEED[cfg])
    outs = []
    for spec in CONFIGS[cfg]:
        if scale_m is not None:
            spec = dataclasses.replace(spec, M=scale_m)
        chained = spec.name.endswith("-down")
        d = make_linear(spec, rng, with_x=not chained)
        d["spec"] = spec
        outs.append(d)
    return outs


def edge_tensor(kind: str, rows: int, cols: int, seed: int = 7) -> np.ndarray:
    """Deterministic bf16 bit tensors that hit quantizer corner cases.

    kinds: zeros, negzeros, subnormal (bf16 subnormals and tiny normals),
    ties (block maxima that make ratios land on E2M1 rounding midpoints),
    huge (values near the bf16 maximum), mixed (per-block mix of the above
    plus random normals with wide exponent spread).
    """
    rng = np.random.default_rng(seed)
    if kind == "zeros":
        return np.zeros((rows, cols), np.uint16)
    if kind == "negzeros":
        b = np.zeros((rows, cols), np.uint16)
        b[rng.random((rows, cols)) < 0.5] = 0x8000
        return b
    if kind == "subnormal":
        mant = rng.integers(0, 128, size=(rows, cols), dtype=np.uint16)
        expo = rng.integers(0, 3, size=(rows, cols), dtype=np.uint16)  # 0 => subnormal
        sign = (rng.random((rows, cols)) < 0.5).astype(np.uint16) << 15
        return sign | (expo << 7) | mant
    if kind == "ties":
        # every block's maximum is 6 * 2^e, so with power-of-two scales the
        # remaining values are exact multiples of quarter steps of the grid
        grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5,
                         2.0, 3.0, 4.0, 6.0, 0.125, 5.5], dtype=np.float32)
        v = grid[rng.integers(0, len(grid), size=(rows, cols))]
        v[::16, ::16] = 6.0
        e = rng.integers(-6, 6, size=(rows // 16, cols // 16)).astype(np.float32)
        v = v * np.repeat(np.repeat(np.exp2(e), 16, 0), 16, 1)
        v[rng.random((rows, cols)) < 0.5] *= -1
        return f32_to_bf16_bits(v)
    if kind == "huge":
        mant = rng.integers(0, 128, size=(rows, cols), dtype=np.uint16)
        expo = rng.integers(240, 255, size=(rows, cols), dtype=np.uint16)
        sign = (rng.random((rows, cols)) < 0.5).astype(np.uint16) << 15
        return sign | (expo << 7) | mant
    if kind == "mixed":
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        e = rng.integers(-40, 40, size=(rows, cols)).astype(np.float32)
        x *= np.exp2(e)
        b = f32_to_bf16_bits(x)
        br, bc = rows // 16, cols // 16
        pick = rng.integers(0, 5, size=(br, bc))
        for i in range(br):
            for j in range(bc):
                blk = (slice(16 * i, 16 * i + 16), slice(16 * j, 16 * j + 16))
                if pick[i, j] == 0:
                    b[blk] = 0
                elif pick[i, j] == 1:
                    b[blk] = edge_tensor("subnormal", 16, 16, seed + 31 * i + j)
                elif pick[i, j] == 2:
                    b[blk] = edge_tensor("ties", 16, 16, seed + 17 * i + j)
        return b
    raise ValueError(kind)
