#!/usr/bin/env python3
"""Benchmark of the W4A4G4 triple-branch linear on one MI355X.

One step = the whole hot path of one linear, forward and backward, on the
FLUX MLP-up shape X[4608 x 3072] -> Y[4608 x 12288] (stabilizer rank 32,
LoRA rank 16, Student-t activations):

  Q(X) -> T = X [L1 | A] -> Y = Q(X) Q(R)^T + T [L2; B]           (forward)
  Q(G) -> V = G [L2; B]^T -> dX = Q(G) Q(R) + V [L1 | A]^T,
                              dA = X^T V_A, dB = T_A^T G           (backward)

Q(R) is prepared once (R is frozen) and is not part of the step.  Inputs are
resident in HBM before timing starts.  `value` is 4*M*N*K (the fwd + dX 4-bit
GEMM work; the low-rank FLOPs are not counted) divided by the step time.

Prints one JSON line.  --gpus N with N > 1 is refused: the library runs the hot path on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 (and MXFP6), published
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="token rows of the oracle sample (0: all)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle passes over the sample")
    ap.add_argument("--quant-reps", type=int, default=20)
    ap.add_argument("--path", choices=["fused", "codes", "op"], default="fused",
                    help="fused: one pass quantizes and down-projects X (and G), GEMMs read E2M1 codes; "
                         "codes: separate quantizer and low-rank passes; op: pair-merged FP6 GEMM operands")
    ap.add_argument("--prewarm-ms", type=float, default=250.0,
                    help="GPU time of untimed steps before the counted warm-up (clocks settle)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config block")
    ap.add_argument("--config-reps", type=int, default=10)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 512 MiB device copy (counter calibration for profiles)")
    return ap.parse_args()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def make_inputs():
    import synth
    spec = synth.CONFIGS["c3"][0]          # the MLP-up linear of the MLP pair config
    rng = np.random.default_rng(synth.CONFIG_SEED["c3"])
    d = synth.make_linear(spec, rng)
    return spec, d


N_INPUT_SETS = 3   # X, G sets the timed steps rotate through (inputs of a step: 141 MB each)


def extra_inputs(spec, d, n):
    """n - 1 further (X, G) pairs drawn like the first (same distributions, the
    same outlier columns of X), so that consecutive steps read different inputs
    and the three sets (423 MB) exceed the 256 MB MALL, as new batches would."""
    import synth
    out = []
    for i in range(1, n):
        rng = np.random.default_rng(synth.CONFIG_SEED["c3"] + 1000 + i)
        X = synth.make_tensor(rng, (spec.M, spec.K), spec.x_dist)
        cols = d["x_outlier_cols"]
        if len(cols):
            X[:, cols] *= np.float32(spec.x_outlier_mult)
        G = synth.make_tensor(rng, (spec.M, spec.N), "normal", spec.g_std)
        out.append((synth.f32_to_bf16_bits(X), synth.f32_to_bf16_bits(G)))
    return out


class Linear:
    """Device buffers and the step of one triple-branch linear (all preallocated).

    path "fused": one pass over X (G) writes Q(X) (Q(G)) and T (V); the GEMMs
    read E2M1 codes + scales.  path "codes": the same with separate quantizer and
    low-rank passes.  path "op": the quantizer writes the pair-merged operands
    and the GEMMs read them (a full 32-K fragment per MFMA)."""

    def __init__(self, spec, d, path="op", more_inputs=(), fold_db=False):
        import torch
        from bit_quantized_lora_amd import ops
        self.ops, self.path, self.fold_db = ops, path, fold_db and path == "fused"
        M, K, N, rs, r = spec.M, spec.K, spec.N, spec.rs, spec.r
        self.M, self.K, self.N = M, K, N
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        self.X, self.G = dev_bf16(d["X"]), dev_bf16(d["G"])
        self.inputs = [(self.X, self.G)] + [(dev_bf16(x), dev_bf16(g)) for x, g in more_inputs]
        self.k = 0
        self.L1t = dev_bf16(np.ascontiguousarray(d["L1"].T))
        self.At = dev_bf16(np.ascontiguousarray(d["A"].T))
        self.L2, self.B = dev_bf16(d["L2"]), dev_bf16(d["B"])
        R = dev_bf16(d["R"])
        # offline: Q(R) (R is frozen)
        if path == "op":
            self.ro = ops.quant_block16_op(R, op_rm=True, op_cm=True)
            (a, b), (c, dd) = ops.operand_shapes(M, K)
            self.xo = {"op_rm": e((a, b), u8), "op_rm_scales": e((c, dd), u8)}
            (a, b), (c, dd) = ops.operand_shapes(M, N)
            self.go = {"op_rm": e((a, b), u8), "op_rm_scales": e((c, dd), u8)}
        else:
            self.rq, self.rqc, self.rs_, self.rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
            self.xq = (e((M, K // 2), u8), None, e((M // 16, K // 16), u8))
            self.gq = (e((M, N // 2), u8), None, e((M // 16, N // 16), u8))
        self.R = R
        self.T, self.V = e((M, rs + r), f32), e((M, rs + r), f32)
        self.Y, self.dX = e((M, N), bf), e((M, K), bf)
        self.dAt, self.dB = e((r, K), f32), e((r, N), f32)
        self.ws = e((max(ops.linear_bwd_workspace(M, N, K, r), 16),), u8)
        self.ws_lr = e((max(ops.lowrank_workspace(M, K, rs + r), ops.lowrank_workspace(M, N, rs + r), 16),), u8)
        # the step's library calls, checked once per input set and issued as prepared
        # calls (no per-step Python checks); a layer whose X or G is replaced (a
        # chained layer) falls back to the ordinary calls
        self.p_fwd = self.p_qx = self.p_qg = self.p_bwd = None
        if path != "op":
            self.p_fwd = ops.linear_fwd(self.xq[0], self.xq[2], self.rq, self.rs_, self.T, self.L2, self.B, M, N, K,
                                        out=self.Y, prepare=True)
            self.p_bwd = [ops.linear_bwd(self.gq[0], self.gq[2], self.rqc, self.rsct, self.V, self.L1t, self.At,
                                         x, g, self.T, M, N, K, workspace=self.ws, dX=self.dX, dAt=self.dAt,
                                         dB=self.dB, prepare=True, skip_dB=self.fold_db) for x, g in self.inputs]
        if path == "fused":
            self.p_qx = [ops.quant_lowrank(x, self.L1t, self.At, out=self.T, codes=self.xq[0], scales=self.xq[2],
                                           workspace=self.ws_lr, prepare=True) for x, _ in self.inputs]
            if self.fold_db:   # dB = (X A)^T G taken in the pass over G
                self.ws_db = e((ops.quant_lowrank_db_workspace(M, N, rs + r, r),), u8)
                self.p_qg = [ops.quant_lowrank_db(g, self.L2, self.B, self.T, out=self.V, codes=self.gq[0],
                                                  scales=self.gq[2], dB=self.dB, workspace=self.ws_db, prepare=True)
                             for _, g in self.inputs]
            else:
                self.p_qg = [ops.quant_lowrank(g, self.L2, self.B, out=self.V, codes=self.gq[0], scales=self.gq[2],
                                               workspace=self.ws_lr, prepare=True) for _, g in self.inputs]

    def _own_inputs(self):
        return self.X is self.inputs[self.k][0] and self.G is self.inputs[self.k][1]

    def quant_lowrank_x(self):
        if self.path == "fused" and self.X is self.inputs[self.k][0]:
            self.p_qx[self.k]()
        elif self.path == "fused":
            self.ops.quant_lowrank(self.X, self.L1t, self.At, out=self.T, codes=self.xq[0], scales=self.xq[2],
                                   workspace=self.ws_lr)
        else:
            self.quant_x()
            self.lowrank_x()

    def quant_lowrank_g(self):
        if self.path == "fused" and self.G is self.inputs[self.k][1]:
            self.p_qg[self.k]()
        elif self.path == "fused":
            self.ops.quant_lowrank(self.G, self.L2, self.B, out=self.V, codes=self.gq[0], scales=self.gq[2],
                                   workspace=self.ws_lr)
        else:
            self.quant_g()
            self.lowrank_g()

    def quant_x(self):
        if self.path == "op":
            self.ops.quant_block16_op(self.X, op_rm=True, out=self.xo)
        else:
            self.ops.quant_block16(self.X, out=self.xq)

    def lowrank_x(self):
        self.ops.lowrank_fused(self.X, self.L1t, self.At, out=self.T, workspace=self.ws_lr)

    def gemm_fwd(self):
        o, M, N, K = self.ops, self.M, self.N, self.K
        if self.path == "op":
            o.linear_fwd_op(self.xo["op_rm"], self.xo["op_rm_scales"], self.ro["op_rm"], self.ro["op_rm_scales"],
                            self.T, self.L2, self.B, M, N, K, out=self.Y)
        else:
            self.p_fwd()

    def quant_g(self):
        if self.path == "op":
            self.ops.quant_block16_op(self.G, op_rm=True, out=self.go)
        else:
            self.ops.quant_block16(self.G, out=self.gq)

    def lowrank_g(self):
        self.ops.lowrank_fused(self.G, self.L2, self.B, out=self.V, workspace=self.ws_lr)

    def gemm_bwd_and_grads(self):
        o, M, N, K = self.ops, self.M, self.N, self.K
        if self.path == "op":
            o.linear_bwd_op(self.go["op_rm"], self.go["op_rm_scales"], self.ro["op_cm"], self.ro["op_cm_scales"],
                            self.V, self.L1t, self.At, self.X, self.G, self.T, M, N, K, workspace=self.ws,
                            dX=self.dX, dAt=self.dAt, dB=self.dB)
        elif self._own_inputs():
            self.p_bwd[self.k]()
        else:
            o.linear_bwd(self.gq[0], self.gq[2], self.rqc, self.rsct, self.V, self.L1t, self.At, self.X, self.G,
                         self.T, M, N, K, workspace=self.ws, dX=self.dX, dAt=self.dAt, dB=self.dB)

    def forward(self):
        self.quant_lowrank_x()
        self.gemm_fwd()

    def backward(self):
        self.quant_lowrank_g()
        self.gemm_bwd_and_grads()

    def next_inputs(self):
        """The next (X, G) set (host-side reference swap, no device work)."""
        self.k = (self.k + 1) % len(self.inputs)
        self.X, self.G = self.inputs[self.k]

    def step(self):
        self.next_inputs()
        self.forward()
        self.backward()


def time_quantizer(reps, c4):
    """Standalone quantizer (both code layouts, E8M0 scales) over the QKV config's
    own X [18432 x 3072] and dY [18432 x 9216], rotating copies in distinct
    buffers that together exceed the 256 MB MALL; beside it, in the same run, a
    plain streaming kernel over the same buffers with the same 2 : 1 read : write
    bytes (ft_stream_2to1: 2 B read, 1 B written per element)."""
    import torch
    from bit_quantized_lora_amd import ops
    out = {}
    for name, bits, ncopies in (("X", c4["X"], 3), ("dY", c4["G"], 2)):
        rows, cols = bits.shape
        x0 = dev_bf16(bits)
        xs = [x0] + [x0.clone() for _ in range(ncopies - 1)]
        bufs = [ops.quant_block16(x, rm=True, cm=True) for x in xs]
        sink = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda") for _ in range(ncopies)]
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()

        def timed(fn):
            prewarm(lambda: fn(0), SECTION_WARM_MS)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for i in range(reps):
                fn(i)
            e1.record(s)
            e1.synchronize()
            return e0.elapsed_time(e1) / 1e3 / reps

        sec = timed(lambda i: ops.quant_block16(xs[i % ncopies], rm=True, cm=True, out=bufs[i % ncopies]))
        sec_stream = timed(lambda i: ops.stream_2to1(xs[i % ncopies], sink[i % ncopies]))
        elems = rows * cols
        alg_bytes = elems * 2 + elems // 2 * 2 + elems // 256   # bf16 in, two code layouts, E8M0 scales
        out[name] = {"shape": [rows, cols], "us": sec * 1e6, "GBps": alg_bytes / sec / 1e9,
                     "bytes_per_elem": alg_bytes / elems,
                     "streaming_ref_us": sec_stream * 1e6, "streaming_ref_GBps": 3 * elems / sec_stream / 1e9,
                     "frac_of_streaming_ref": (alg_bytes / sec) / (3 * elems / sec_stream)}
        del xs, bufs, sink, x0
        torch.cuda.empty_cache()
    return out


def time_mlp_fc1_fusion(lin, reps):
    """The first linear of the MLP pair up to the second linear's inputs -- Y, h =
    GELU(Y), Q(h) and T_down = h [L1_down | A_down] -- with the MLP fusion in the
    GEMM epilogue (it writes Y, h and Q(h); one low-rank pass over h), with the
    MLP fusion in the second linear's input pass (GEMM, then one pass over Y
    writing h, Q(h) and T_down) and with separate kernels (GEMM, GELU, one
    quantize + low-rank pass over h).  Down factors are
    seeded random bf16 of the MLP-down shape (rs 32, r 16)."""
    import torch
    from bit_quantized_lora_amd import ops
    if lin.path == "op":
        return None
    M, N, K = lin.M, lin.N, lin.K
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1002)
    wa = (0.02 * torch.randn(32, N, device="cuda", generator=gen)).to(torch.bfloat16)
    wb = (0.01 * torch.randn(16, N, device="cuda", generator=gen)).to(torch.bfloat16)
    bf, u8 = torch.bfloat16, torch.uint8
    Y, H = torch.empty((M, N), dtype=bf, device="cuda"), torch.empty((M, N), dtype=bf, device="cuda")
    hc, hs = torch.empty((M, N // 2), dtype=u8, device="cuda"), torch.empty((M // 16, N // 16), dtype=u8, device="cuda")
    Td = torch.empty((M, 48), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(ops.lowrank_workspace(M, N, 48), 16),), dtype=u8, device="cuda")
    xq, xs = lin.xq[0], lin.xq[2]

    def fused():
        ops.linear_fwd_gelu(xq, xs, lin.rq, lin.rs_, lin.T, lin.L2, lin.B, M, N, K, out=(Y, H, hc, hs))
        ops.lowrank_fused(H, wa, wb, out=Td, workspace=ws)

    def separate():
        ops.linear_fwd(xq, xs, lin.rq, lin.rs_, lin.T, lin.L2, lin.B, M, N, K, out=Y)
        ops.gelu_fwd(Y, out=H)
        ops.quant_lowrank(H, wa, wb, out=Td, codes=hc, scales=hs, workspace=ws)

    def fused_pass():   # GELU, Q(h) and T_down in the pass that reads Y once
        ops.linear_fwd(xq, xs, lin.rq, lin.rs_, lin.T, lin.L2, lin.B, M, N, K, out=Y)
        ops.gelu_quant_lowrank(Y, wa, wb, out=(H, Td, hc, hs), workspace=ws)

    res = {}
    s = torch.cuda.current_stream()
    for name, fn in (("fused_us", fused), ("fused_pass_us", fused_pass), ("separate_us", separate)):
        prewarm(fn, SECTION_WARM_MS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        e1.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    res["speedup"] = round(res["separate_us"] / res["fused_us"], 3)
    res["speedup_fused_pass"] = round(res["separate_us"] / res["fused_pass_us"], 3)
    return res


def time_precision_variants(lin, reps):
    """The precision settings of the paper's Table 4 on the same linear: the bf16
    x E2M1 GEMMs (W4A16 forward: X unquantized; G16 backward: G unquantized)
    against the 4-bit ones, each launched back to back, and the whole fwd+bwd
    step of each setting (an A16 / G16 side skips its quantizer but keeps the
    low-rank pass)."""
    import torch
    from bit_quantized_lora_amd import ops
    if lin.path == "op":
        return None
    M, N, K = lin.M, lin.N, lin.K
    Yv, dXv = torch.empty_like(lin.Y), torch.empty_like(lin.dX)
    dAt, dB = torch.empty_like(lin.dAt), torch.empty_like(lin.dB)

    def fwd_a16():
        ops.linear_fwd_a16(lin.X, lin.rq, lin.rs_, lin.T, lin.L2, lin.B, M, N, K, out=Yv)

    def bwd_g16():
        ops.linear_bwd_g16(lin.G, lin.rqc, lin.rsct, lin.V, lin.L1t, lin.At, lin.X, lin.T, M, N, K,
                           workspace=lin.ws, dX=dXv, dAt=dAt, dB=dB)

    def step(a16, g16):
        def run():
            if a16:
                lin.lowrank_x()
                fwd_a16()
            else:
                lin.forward()
            if g16:
                lin.lowrank_g()
                bwd_g16()
            else:
                lin.backward()
        return run

    s = torch.cuda.current_stream()

    def timed(fn):
        prewarm(fn, SECTION_WARM_MS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    flops = 2.0 * M * N * K
    res = {}
    for name, fn in (("fwd_gemm_w4a4", lin.gemm_fwd), ("fwd_gemm_w4a16", fwd_a16),
                     ("bwd_w4g4", lin.gemm_bwd_and_grads), ("bwd_g16", bwd_g16)):
        us = timed(fn)
        res[name] = {"us": round(us, 2), "TFLOPs": round(flops / us / 1e6, 1)}
    res["fwd_gemm_w4a16"]["frac_bf16_peak"] = round(res["fwd_gemm_w4a16"]["TFLOPs"] / BF16_PEAK_TFLOPS, 4)
    res["step_us"] = {tag: round(timed(step(a16, g16)), 2)
                      for tag, a16, g16 in (("W4A4G4", False, False), ("W4A16G4", True, False),
                                            ("W4A4G16", False, True), ("W4A16G16", True, True))}
    return res


_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _deq(codes, scales, bh, bw):
    """fp64 values of packed row-major E2M1 codes with E8M0 scales over bh x bw
    blocks (measurement helper: quantization error of the GPU quantizers)."""
    import torch
    lut = torch.tensor(_E2M1, dtype=torch.float64, device=codes.device)
    c = codes.to(torch.int64)
    vals = torch.stack([lut[c & 15], lut[c >> 4]], dim=-1).reshape(codes.shape[0], -1)
    sc = torch.exp2(scales.to(torch.float64) - 127.0)
    return vals * sc.repeat_interleave(bh, 0).repeat_interleave(bw, 1)


def time_granularity(lin, reps):
    """The quantization granularities of the paper's Table 5 on the benchmark
    linear: relative quantization MSE of X, R, G and of the backward's operand
    for R^T, and the time of each 4-bit step.  16x16: the method (Q(R)^T read in
    place).  1 x g groups (g = 16, 32): forward GEMM, backward GEMM + adapter
    gradients, and the re-quantization Q_g(deq(Q_g(R))^T) the transposed product
    needs (a pass over R per step, or a second stored copy of the weight)."""
    import torch
    from bit_quantized_lora_amd import ops
    if lin.path == "op":
        return None
    M, N, K = lin.M, lin.N, lin.K
    s = torch.cuda.current_stream()

    def timed(fn):
        prewarm(fn, SECTION_WARM_MS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        e1.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / reps, 2)

    def rel_mse(ref, deq):
        ref = ref.to(torch.float64)
        return float(((ref - deq) ** 2).sum() / (ref ** 2).sum())

    X, R, G = lin.X, lin.R, lin.G
    out = {}
    xq, _, xs = ops.quant_block16(X)
    gq, _, gs = ops.quant_block16(G)
    out["16x16"] = {
        "mse_X": rel_mse(X, _deq(xq, xs, 16, 16)), "mse_R": rel_mse(R, _deq(lin.rq, lin.rs_, 16, 16)),
        "mse_G": rel_mse(G, _deq(gq, gs, 16, 16)),
        "mse_Rt_operand": rel_mse(R.t(), _deq(lin.rqc, lin.rsct, 16, 16)),
        "fwd_gemm_us": timed(lin.gemm_fwd), "bwd_us": timed(lin.gemm_bwd_and_grads), "requant_Rt_us": 0.0}
    dX, dAt, dB = torch.empty_like(lin.dX), torch.empty_like(lin.dAt), torch.empty_like(lin.dB)
    Y = torch.empty_like(lin.Y)
    for g in (16, 32):
        xq, xs = ops.quant_group(X, g)
        rq, rsc = ops.quant_group(R, g)
        gq, gs = ops.quant_group(G, g)
        rtq, rts = ops.requant_group_t(rq, rsc, N, K, g)
        direct_q, direct_s = ops.quant_group(R.t().contiguous(), g)
        rec = {"mse_X": rel_mse(X, _deq(xq, xs, 1, g)), "mse_R": rel_mse(R, _deq(rq, rsc, 1, g)),
               "mse_G": rel_mse(G, _deq(gq, gs, 1, g)),
               "mse_Rt_operand": rel_mse(R.t(), _deq(rtq, rts, 1, g)),
               "mse_Rt_if_quantized_from_R": rel_mse(R.t(), _deq(direct_q, direct_s, 1, g))}
        rec["fwd_gemm_us"] = timed(lambda: ops.linear_fwd_grp(g, xq, xs, rq, rsc, lin.T, lin.L2, lin.B, M, N, K,
                                                              out=Y))
        rec["bwd_us"] = timed(lambda: ops.linear_bwd_grp(g, gq, gs, rtq, rts, lin.V, lin.L1t, lin.At, lin.X, lin.G,
                                                         lin.T, M, N, K, workspace=lin.ws, dX=dX, dAt=dAt, dB=dB))
        rec["requant_Rt_us"] = timed(lambda: ops.requant_group_t(rq, rsc, N, K, g, out=(rtq, rts)))
        rec["quant_X_us"] = timed(lambda: ops.quant_group(X, g, out=(xq, xs)))
        out[f"1x{g}"] = rec
        del direct_q, direct_s
    flops = 2.0 * M * N * K
    for v in out.values():
        for k in list(v):
            if k.startswith("mse"):
                v[k] = float(f"{v[k]:.4e}")
        v["fwd_gemm_TFLOPs"] = round(flops / v["fwd_gemm_us"] / 1e6, 1)
        v["fwd_gemm_frac_fp4_peak"] = round(flops / v["fwd_gemm_us"] / 1e6 / FP4_PEAK_TFLOPS, 4)
    return out


def time_separate_passes(spec, d, more, steps, warmup, one_pass_us):
    """The same linear step with the quantizer and the shared down-projection as
    separate kernels (path "codes"), against the one-pass default: the layer-level
    effect of folding Q(in) into the low-rank pass."""
    import torch
    lin = Linear(spec, d, "codes", more)
    for _ in range(warmup):
        lin.step()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        lin.step()
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del lin
    return {"step_us_one_pass": round(one_pass_us, 2), "step_us_separate_passes": round(us, 2),
            "speedup": round(us / one_pass_us, 3)}


def time_graph_step(lin, steps):
    """The same step captured once per input set in a HIP graph (torch.cuda.CUDAGraph)
    and replayed in rotation: GPU time per step and the host's time to enqueue one
    replay, against the eager calls' host time.  None on the pair-merged path."""
    import torch
    if lin.path == "op":
        return None
    s = torch.cuda.current_stream()
    graphs = []
    for _ in range(len(lin.inputs)):   # each capture takes the next input set
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lin.step()
        graphs.append(g)
    torch.cuda.synchronize()
    k = [0]

    def replay():
        graphs[k[0] % len(graphs)].replay()
        k[0] += 1
    prewarm(replay, SECTION_WARM_MS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    h0 = time.perf_counter()
    for _ in range(steps):
        replay()
    host_us = (time.perf_counter() - h0) / steps * 1e6
    e1.record(s)
    e1.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / steps, 4), "host_enqueue_us_per_step": round(host_us, 1),
            "graphs": len(graphs)}


def time_db_fold(spec, d, more, steps, warmup, default_us):
    """The same linear step with dB = (X A)^T G folded into the backward's pass
    over G (ft_quant_lowrank_db, then ft_linear_bwd without dB) against the
    default, where dB is taken, beside the dX GEMM, by the extra workgroups of its
    launch."""
    import torch
    lin = Linear(spec, d, "fused", more, fold_db=True)
    for _ in range(warmup):
        lin.step()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        lin.step()
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the G pass alone, each way
    ph = {}
    for name, fn in (("g_pass_with_db", lin.quant_lowrank_g),):
        prewarm(fn, SECTION_WARM_MS)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(s)
        for _ in range(steps):
            fn()
        g1.record(s)
        g1.synchronize()
        ph[name] = round(g0.elapsed_time(g1) * 1e3 / steps, 2)
    del lin
    return {"step_us_default_dB_beside_dX_gemm": round(default_us, 2), "step_us_dB_in_G_pass": round(us, 2),
            "speedup": round(default_us / us, 3), **ph}


def lowrank_pass_rates(spec, phases):
    """HBM roofline of the one-pass quantize + down-projection (in the step's
    phase times, split sum included): algorithmic bytes = bf16 input read, E2M1
    codes and E8M0 scales written, the fp32 projection written."""
    M, K, N, rho = spec.M, spec.K, spec.N, spec.rs + spec.r
    out = {}
    for name, kin, key in (("X", K, "quant_lowrank_X"), ("G", N, "quant_lowrank_G")):
        alg = 2 * M * kin + M * kin // 2 + M * kin // 256 + 4 * M * rho
        us = phases[key]
        out[name] = {"us": round(us, 2), "alg_MB": round(alg / 1e6, 1), "GBps": round(alg / us / 1e3, 1),
                     "frac_hbm": round(alg / us / 1e3 / HBM_PEAK_GBPS, 4)}
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a4_fwd_mlp_up.traffic.txt")
GEMM_SRCS = [os.path.join(ROOT, "bit_quantized_lora_amd", "csrc", f) for f in ("gemm_w4a4.hip", "gemm_tile.h")]


def measured_traffic():
    """HBM bytes per forward-GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE x calibration + WRITE_SIZE), or None if the kernel source changed since."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(b"".join(open(p, "rb").read() for p in GEMM_SRCS)).hexdigest()
    if kv.get("gemm_source_sha256") != sha:
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def calibration_copy():
    import torch
    src = torch.ones(256 << 20, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def _layer(d):
    """A prepared fused-path Linear for one linear of a config (a chained second
    linear of a pair gets its X from the first linear's GELU at run time)."""
    spec = d["spec"]
    if "X" not in d:
        d = dict(d)
        d["X"] = np.zeros((spec.M, spec.K), np.uint16)
    return Linear(spec, d, "fused")


def _oracle_sample_s(d, rows):
    """Seconds the oracle takes for one linear's fwd + bwd over its first `rows`
    tokens (Q(R) prepared outside the timing), and the token count."""
    import oracle as O
    spec = d["spec"]
    rows = min(rows, spec.M)
    X = d["X"][:rows] if "X" in d else np.zeros((rows, spec.K), np.uint16)
    G = d["G"][:rows]
    f = {k: O.bf16_to_f64(d[k]) for k in ("L1", "L2", "A", "B")}
    rc, rsc = O.quantize_block16(d["R"])
    Rhat = O.dequantize(rc, rsc, "pow2")
    t0 = time.perf_counter()
    xc, xs = O.quantize_block16(X); gc, gs = O.quantize_block16(G)
    Xf, Gf = O.bf16_to_f64(X), O.bf16_to_f64(G)
    O.linear_fwd(O.dequantize(xc, xs, "pow2"), Rhat, Xf, f["L1"], f["L2"], f["A"], f["B"])
    O.linear_bwd(O.dequantize(gc, gs, "pow2"), Rhat, Gf, Xf, f["L1"], f["L2"], f["A"], f["B"])
    return time.perf_counter() - t0, rows


def time_configs(reps, cache, oracle_rows=128):
    """Per-config block: every config of the workload list on the fused path.

    c1, c2, c4: one linear, fwd + bwd.  c3: the MLP pair chained (up -> GELU ->
    down forward, then down, GELU and up backward).  c5: the double-stream
    block's eight linears (per stream: qkv and proj on their own inputs, up ->
    GELU -> down chained).  Reported: step time (median over `reps` steps),
    4-bit GEMM work of the step per second and its fraction of the FP4 peak, each
    linear's forward GEMM and its backward call (dX GEMM with the adapter
    gradients) alone, launched back to back, the quantizer's rate on
    the config's first input, and the oracle's time on a bounded sample of every
    linear (the first `oracle_rows` tokens, scaled to the full token count)."""
    import torch
    import synth
    from bit_quantized_lora_amd import ops
    s = torch.cuda.current_stream()
    out = {}
    for cfg in ("c1", "c2", "c3", "c4", "c5"):
        ds = cache[cfg] if cfg in cache else synth.config_linears(cfg)
        lins = {d["spec"].name: _layer(d) for d in ds}
        singles = [n for n in lins if not (n.endswith("-up") or n.endswith("-down"))]
        pairs = [(n, n[:-3] + "-down") for n in lins if n.endswith("-up")]
        bufs = {u: (torch.empty_like(lins[u].Y), torch.empty_like(lins[u].Y)) for u, _ in pairs}

        def step():
            for n in singles:
                lins[n].forward()
                lins[n].backward()
            for u, dn in pairs:
                up, down = lins[u], lins[dn]
                h, dy = bufs[u]
                up.forward()
                ops.gelu_fwd(up.Y, out=h)
                down.X = h
                down.forward()
                down.backward()
                ops.gelu_bwd(up.Y, down.dX, out=dy)
                up.G = dy
                up.backward()

        prewarm(step, SECTION_WARM_MS)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(s)
        for i in range(reps):
            step()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        step_us = float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]))
        work = sum(4.0 * l.M * l.N * l.K for l in lins.values())
        gemms = {}
        for n, lin in lins.items():
            for _ in range(2):
                lin.gemm_fwd()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(s)
            for _ in range(reps):
                lin.gemm_fwd()
            g1.record(s)
            g1.synchronize()
            us = g0.elapsed_time(g1) * 1e3 / reps
            tf = 2.0 * lin.M * lin.N * lin.K / us / 1e6
            gemms[n] = {"us": round(us, 2), "TFLOPs": round(tf, 1), "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
        bwds = {}   # ft_linear_bwd alone: the dX GEMM with the adapter gradients (TFLOP/s of the dX GEMM's 2MNK)
        for n, lin in lins.items():
            for _ in range(2):
                lin.gemm_bwd_and_grads()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(s)
            for _ in range(reps):
                lin.gemm_bwd_and_grads()
            g1.record(s)
            g1.synchronize()
            us = g0.elapsed_time(g1) * 1e3 / reps
            tf = 2.0 * lin.M * lin.N * lin.K / us / 1e6
            bwds[n] = {"us": round(us, 2), "TFLOPs": round(tf, 1), "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
        first = lins[ds[0]["spec"].name]
        q = ops.quant_block16(first.X, rm=True, cm=True)
        for _ in range(2):
            ops.quant_block16(first.X, rm=True, cm=True, out=q)
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(s)
        for _ in range(reps):
            ops.quant_block16(first.X, rm=True, cm=True, out=q)
        q1.record(s)
        q1.synchronize()
        qus = q0.elapsed_time(q1) * 1e3 / reps
        el = first.M * first.K
        qbytes = el * 2 + el + el // 256
        orc_s = 0.0
        for d in ds:
            t, rows = _oracle_sample_s(d, oracle_rows)
            orc_s += t * d["spec"].M / rows
        out[cfg] = {
            "linears": len(lins), "step_us": round(step_us, 2),
            "step_TFLOPs": round(work / step_us / 1e6, 1),
            "step_frac_fp4_peak": round(work / step_us / 1e6 / FP4_PEAK_TFLOPS, 4),
            "fwd_gemm": gemms,
            "bwd_dX_gemm_with_adapter_grads": bwds,
            "quantizer": {"shape": [first.M, first.K], "us": round(qus, 2), "GBps": round(qbytes / qus / 1e3, 1),
                          "note": "repeated on one input (partly served from the MALL when it fits)"},
            "oracle_s_full_est": round(orc_s, 2),
            "oracle_sample": f"first {oracle_rows} tokens of each linear, scaled to the full token count",
        }
        del lins, bufs, q
        torch.cuda.empty_cache()
    return out


class GpuClock:
    """Graphics clock (MHz) of the GPU this process runs on, found among the
    node's GPUs by its PCI address.  The library is opened and the GPU found at
    construction, so that read() is a single query, quick enough to land while
    the GPU is still working through enqueued steps.  read() gives None when the
    tool is missing or the GPU cannot be matched."""

    def __init__(self):
        self.h, self.bdf, self.mod = None, None, None
        try:
            import amdsmi
            import torch
            p = torch.cuda.get_device_properties(torch.cuda.current_device())
            self.bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            amdsmi.amdsmi_init()
            self.mod = amdsmi
            self.h = amdsmi.amdsmi_get_processor_handle_from_bdf(self.bdf)
        except Exception:  # pragma: no cover - tool missing, no permission, or no match
            self.h = None

    def read(self):
        if self.h is None:
            return None
        try:
            t0 = time.perf_counter()
            info = self.mod.amdsmi_get_clock_info(self.h, self.mod.AmdSmiClkType.GFX)
            return {"cur": info.get("clk"), "max": info.get("max_clk"), "bdf": self.bdf,
                    "query_ms": round((time.perf_counter() - t0) * 1e3, 2)}
        except Exception:  # pragma: no cover
            return None

    def close(self):
        if self.mod is not None:
            try:
                self.mod.amdsmi_shut_down()
            except Exception:  # pragma: no cover
                pass
            self.mod = None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# every side measurement first runs its own call for this long: a section that
# follows host-side set-up (new inputs, another section's allocations) finds
# the GPU clock lowered, and three warm-up calls do not bring it back up
SECTION_WARM_MS = 60.0


def prewarm(fn, min_ms=250.0):
    """Run `fn` (one step) until at least min_ms of GPU work has completed, so the
    clocks have settled before the counted warm-up and the timed steps."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return {"steps": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def cpu_baseline(spec, d, rows, reps):
    """The oracle as it stands, `reps` passes over the first `rows` tokens of the same workload."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    rows = rows if 0 < rows <= spec.M else spec.M
    sl = slice(0, rows)
    f = {k: O.bf16_to_f64(d[k]) for k in ("L1", "L2", "A", "B")}
    rc, rsc = O.quantize_block16(d["R"])          # offline prep, outside the timed region
    Rhat = O.dequantize(rc, rsc, "pow2")
    t0 = time.perf_counter()
    for _ in range(reps):
        X = O.bf16_to_f64(d["X"][sl]); G = O.bf16_to_f64(d["G"][sl])
        xc, xs = O.quantize_block16(d["X"][sl]); gc, gs = O.quantize_block16(d["G"][sl])
        Xhat, Ghat = O.dequantize(xc, xs, "pow2"), O.dequantize(gc, gs, "pow2")
        O.linear_fwd(Xhat, Rhat, X, f["L1"], f["L2"], f["A"], f["B"])
        O.linear_bwd(Ghat, Rhat, G, X, f["L1"], f["L2"], f["A"], f["B"])
    sec = time.perf_counter() - t0
    flops = 4.0 * rows * spec.N * spec.K * reps
    # the oracle's quantizer alone (numpy elementwise work: one thread)
    qs = d["X"][:1024]
    q0 = time.perf_counter()
    O.quantize_block16(qs)
    qsec = time.perf_counter() - q0
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "quantizer_1thread_ns_per_elem": round(qsec / qs.size * 1e9, 2),
            "sample": f"fp64 numpy oracle, {reps} passes of fwd+bwd over {rows} of {spec.M} tokens "
                      f"(K={spec.K}, N={spec.N}), Q(R) prepared outside the timing; {sec:.2f} s; "
                      f"cores = the BLAS threads of its products"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: the library runs the hot path on one GPU only; "
                                   "multi-GPU runs are not supported"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    spec, d = make_inputs()
    more = extra_inputs(spec, d, N_INPUT_SETS)
    lin = Linear(spec, d, args.path, more)
    M, K, N = spec.M, spec.K, spec.N
    s = torch.cuda.current_stream()

    # clocks settle over a fixed stretch of steps before the counted warm-up
    warm = prewarm(lin.step, args.prewarm_ms)
    for _ in range(args.warmup):
        lin.step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, no event inside it.  The graphics clock
    # is read while the GPU works through them (after the last step is enqueued,
    # before the synchronize), and the host's enqueue time is recorded.
    clock = GpuClock()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(s)
    h0 = time.perf_counter()
    for i in range(args.steps):
        lin.step()
    host_timed_us = (time.perf_counter() - h0) / args.steps * 1e6
    t_end.record(s)
    clk_during = clock.read()
    torch.cuda.synchronize()
    clock.close()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # per-phase breakdown: events between the phases over `steps` further steps,
    # enqueued back to back so the GPU never waits for the host
    names = ["quant_lowrank_X", "fwd_gemm", "quant_lowrank_G", "bwd_gemm_and_adapter_grads"]
    fns = [lin.quant_lowrank_x, lin.gemm_fwd, lin.quant_lowrank_g, lin.gemm_bwd_and_grads]
    nph = max(args.steps, 20)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(nph)]
    host_t0 = time.perf_counter()
    for k in range(nph):
        lin.next_inputs()
        marks[k][0].record(s)
        for i, f in enumerate(fns):
            f()
            marks[k][i + 1].record(s)
    host_us = (time.perf_counter() - host_t0) / nph * 1e6
    torch.cuda.synchronize()
    phases = {n: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks])) * 1e3 for i, n in enumerate(names)}
    gemm_ms = phases["fwd_gemm"] / 1e3   # the forward GEMM between event markers inside the step
    step_us = np.array([m[0].elapsed_time(m[-1]) * 1e3 for m in marks])
    step_pct = {"p10": round(float(np.percentile(step_us, 10)), 2), "p50": round(float(np.percentile(step_us, 50)), 2),
                "p90": round(float(np.percentile(step_us, 90)), 2)}

    # forward GEMM alone, launched back to back (no event between launches): the
    # per-launch time used for the roofline
    for _ in range(3):
        lin.gemm_fwd()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(s)
    for _ in range(max(args.steps, 20)):
        lin.gemm_fwd()
    g1.record(s)
    torch.cuda.synchronize()
    gemm_b2b_ms = g0.elapsed_time(g1) / max(args.steps, 20)

    separate = (time_separate_passes(spec, d, more, args.steps, args.warmup, ms_step * 1e3)
                if args.path == "fused" else None)
    db_fold = (time_db_fold(spec, d, more, args.steps, args.warmup, ms_step * 1e3)
               if args.path == "fused" else None)
    graph_step = time_graph_step(lin, args.steps)
    mlp_fusion = time_mlp_fc1_fusion(lin, args.steps)
    precision = time_precision_variants(lin, args.steps)
    granularity = time_granularity(lin, args.steps)
    del lin, more
    torch.cuda.empty_cache()
    import synth
    cache = {"c4": synth.config_linears("c4")}
    quant = time_quantizer(args.quant_reps, cache["c4"][0])
    configs = None if args.no_configs else time_configs(args.config_reps, cache)
    if args.calibration_copy:
        calibration_copy()
    gemm_flops = 2.0 * M * N * K
    achieved = gemm_flops / (gemm_b2b_ms / 1e3) / 1e12
    value = 4.0 * M * N * K / (ms_step / 1e3) / 1e12
    rec = {
        "metric": "W4A4G4 linear fwd+bwd TFLOPS & % FP4 peak at 4608x3072x12288; quant GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": "W4A4G4 triple-branch linear fwd+bwd, FLUX MLP-up shape",
                   "M": M, "K": K, "N": N, "stabilizer_rank": spec.rs, "lora_rank": spec.r,
                   "x_dist": "student-t df=3", "scale_rule": "pow2 (amax/6 rounded up to 2^E)",
                   "gemm_operands": ("pair-merged FP6 E3M2 (two 16-K blocks per 32-K MFMA fragment)"
                                     if args.path == "op" else "E2M1 codes (one 16-K block per 32-K fragment)"),
                   "quantizer_and_lowrank": "one pass" if args.path == "fused" else "separate passes",
                   "outputs": "bf16 Y and dX, fp32 dA and dB",
                   "input_sets": f"{N_INPUT_SETS} rotating (X, G) pairs, one per step"},
        "pct_fp4_peak_whole_linear": round(100.0 * value / FP4_PEAK_TFLOPS, 2),
        "roofline": {"kernel": ("gemm_m6_kernel" if args.path == "op" else "gemm_w4a4_kernel") + " (forward)",
                     "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
                     "per_launch_flops": gemm_flops, "avg_launch_us": round(gemm_b2b_ms * 1e3, 2),
                     # the codes path feeds one 16-K block per 32-K MFMA fragment, so its
                     # instruction ceiling is half the FP4 peak
                     "frac_of_half_fragment_ceiling": (round(achieved / (FP4_PEAK_TFLOPS / 2), 4)
                                                       if args.path != "op" else None),
                     "avg_launch_us_in_step": round(gemm_ms * 1e3, 2)},
        "timed_vs_marker_p50": round(ms_step * 1e3 / step_pct["p50"], 4),
        "prewarm": warm,
        "gfx_clock_mhz_during_timed": clk_during,
        "phases_us": {k: round(v, 2) for k, v in phases.items()},
        "step_us_percentiles": step_pct,
        "host_enqueue_us_per_step": round(host_timed_us, 1),
        "host_enqueue_us_per_step_with_phase_markers": round(host_us, 1),
        "quantizer": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in quant.items()},
        "mlp_fc1_fusion_us": mlp_fusion,
        "precision_variants": precision,
        "granularity": granularity,
        "quant_lowrank_pass": lowrank_pass_rates(spec, phases),
        "graph_replay": graph_step,
        "one_pass_vs_separate": separate,
        "dB_in_G_pass_vs_default": db_fold,
        "configs": configs,
        "quant_GBps": round(quant["dY"]["GBps"], 1),
        "quant_frac_hbm": round(quant["dY"]["GBps"] / HBM_PEAK_GBPS, 4),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(spec, d, args.cpu_rows, args.cpu_reps)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
