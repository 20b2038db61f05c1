"""Host-side checks of bench.py: the one-GPU contract, its loud failure without a
GPU, the algorithmic bytes of the one-pass quantize + projection, and the rule
that the committed HBM traffic figure is used only for the GEMM sources it was
measured on."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _run("--gpus", n)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "no GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_quant_lowrank_algorithmic_bytes():
    """bf16 input read (2 B/elt), E2M1 codes (0.5 B/elt) and one E8M0 byte per
    16x16 block written, the fp32 projection [M x rho] written."""
    b = _bench()
    spec = SimpleNamespace(M=4608, K=3072, N=12288, rs=32, r=16)
    res = b.lowrank_pass_rates(spec, {"quant_lowrank_X": 10.0, "quant_lowrank_G": 20.0})
    M, rho = 4608, 48
    for name, kin, us in (("X", 3072, 10.0), ("G", 12288, 20.0)):
        alg = M * kin * 2 + M * kin // 2 + M * kin // 256 + M * rho * 4
        assert res[name]["alg_MB"] == round(alg / 1e6, 1)
        assert res[name]["GBps"] == round(alg / us / 1e3, 1)
        assert res[name]["frac_hbm"] == round(alg / us / 1e3 / 8000.0, 4)


def test_traffic_figure_tied_to_gemm_sources(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source")
    sha = hashlib.sha256(b"kernel source").hexdigest()
    prof = tmp_path / "traffic.txt"
    prof.write_text(f"# comment\ngemm_source_sha256={sha}\nhbm_bytes_per_launch=123456\n")
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(prof))
    monkeypatch.setattr(b, "GEMM_SRCS", [str(src)])
    assert b.measured_traffic() == 123456
    src.write_bytes(b"kernel source, changed")
    assert b.measured_traffic() is None


def test_committed_traffic_profile_names_the_current_sources():
    """The committed summary carries the hash of the GEMM sources it was measured
    on; the bench reports its bytes only while they match."""
    b = _bench()
    kv = dict(l.strip().split("=", 1) for l in open(b.TRAFFIC_FILE) if "=" in l and not l.startswith("#"))
    sha = hashlib.sha256(b"".join(open(p, "rb").read() for p in b.GEMM_SRCS)).hexdigest()
    got = b.measured_traffic()
    if kv["gemm_source_sha256"] == sha:
        assert got == int(float(kv["hbm_bytes_per_launch"]))
    else:
        assert got is None
