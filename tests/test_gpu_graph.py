"""The linear's four library calls (one pass over X, the forward GEMM, one pass
over G, the backward with its adapter gradients on the library's side stream)
captured in a HIP graph through torch.cuda.CUDAGraph and replayed.  Every
replay, with eager calls and synchronizations between the replays, must give
the bits of the same calls issued eagerly: the graph holds kernel nodes and the
side stream's fork and join dependencies only (no memset nodes), and a replay
runs on whatever the captured buffers hold at that time."""
import numpy as np
import pytest

import synth
from gpu_util import dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

# (M, K, N, rs, r): the MLP-up shape of a FLUX block (one GEMM round, side
# stream beside the dX GEMM) and 512 text tokens (128 x 128 tiles and split
# reductions in both GEMMs, so the split partials' workspaces are in the graph)
SHAPES = [(4608, 3072, 12288, 32, 16), (512, 3072, 3072, 32, 32)]


class _Step:
    """Buffers and prepared library calls of one fwd + bwd step of the linear."""

    def __init__(self, M, K, N, rs, r, seed):
        import torch
        from bit_quantized_lora_amd import ops
        spec = synth.LinearSpec("g", M, K, N, rs, r, x_dist="t3", x_outlier_count=4, x_outlier_mult=30.0)
        d = synth.make_linear(spec, np.random.default_rng(seed))
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
        self.X, self.G = dev_bf16(d["X"]), dev_bf16(d["G"])
        R = dev_bf16(d["R"])
        L1t, At = dev_bf16(np.ascontiguousarray(d["L1"].T)), dev_bf16(np.ascontiguousarray(d["A"].T))
        L2, B = dev_bf16(d["L2"]), dev_bf16(d["B"])
        rq, rqc, rsc, rsct = ops.quant_block16(R, rm=True, cm=True, scales_cm=True)
        rho = rs + r
        self.T, self.V = e((M, rho), f32), e((M, rho), f32)
        self.xq, self.xs = e((M, K // 2), u8), e((M // 16, K // 16), u8)
        self.gq, self.gs = e((M, N // 2), u8), e((M // 16, N // 16), u8)
        self.Y, self.dX = e((M, N), bf), e((M, K), bf)
        self.dAt, self.dB = e((r, K), f32), e((r, N), f32)
        ws_lr = e((max(ops.lowrank_workspace(M, K, rho), ops.lowrank_workspace(M, N, rho), 16),), u8)
        ws_f = e((max(ops.linear_fwd_workspace(M, N, K), 16),), u8)
        ws_b = e((max(ops.linear_bwd_workspace(M, N, K, r), 16),), u8)
        self.calls = [
            ops.quant_lowrank(self.X, L1t, At, out=self.T, codes=self.xq, scales=self.xs, workspace=ws_lr,
                              prepare=True),
            ops.linear_fwd(self.xq, self.xs, rq, rsc, self.T, L2, B, M, N, K, out=self.Y, workspace=ws_f,
                           prepare=True),
            ops.quant_lowrank(self.G, L2, B, out=self.V, codes=self.gq, scales=self.gs, workspace=ws_lr,
                              prepare=True),
            ops.linear_bwd(self.gq, self.gs, rqc, rsct, self.V, L1t, At, self.X, self.G, self.T, M, N, K,
                           workspace=ws_b, dX=self.dX, dAt=self.dAt, dB=self.dB, prepare=True),
        ]
        self.outs = {"T": self.T, "xq": self.xq, "xs": self.xs, "Y": self.Y, "V": self.V, "gq": self.gq,
                     "gs": self.gs, "dX": self.dX, "dAt": self.dAt, "dB": self.dB}

    def run(self):
        for c in self.calls:
            c()

    def poison(self):
        """Overwrite every output (eager fills) so a replay has to write them all."""
        import torch
        for t in self.outs.values():
            if t.dtype == torch.uint8:
                t.fill_(0xA5)
            else:
                t.fill_(float("nan"))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_graph_replays_match_eager_calls(shape):
    require_gpu()
    import torch
    M, K, N, rs, r = shape
    say(f"[graph] M={M} K={K} N={N} rs={rs} r={r}")
    step = _Step(M, K, N, rs, r, seed=M + K + N)
    other = _Step(M, K, N, rs, r, seed=M + K + N + 1)   # eager work between the replays
    step.run()
    other.run()
    torch.cuda.synchronize()
    ref = {k: host(v).copy() for k, v in step.outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # settle on a side stream before the capture
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for rep in range(3):
        step.poison()
        other.run()
        torch.cuda.synchronize()
        g.replay()
        if rep == 1:
            other.run()   # eager calls queued behind a replay
        torch.cuda.synchronize()
        for k, v in step.outs.items():
            got = host(v)
            assert np.array_equal(got.view(np.uint8), ref[k].view(np.uint8)), f"replay {rep}: {k} differs"
    say(f"[graph] 3 replays identical to the eager calls ({len(ref)} outputs)")
