"""Host-side logic of bench.py, on the CPU (no GPU): the one-GPU refusal, the
half-tile rule it shares with the library's launcher, the traffic summary's tie to
the GEMM source, and the step's algorithmic FLOP count."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402

DOMINANT = "fp8k::gemm_tn_kernel<1, 0, false, 0, false, false, true>"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_half_tile_kernel_name():
    assert bench.half_tile_kernel(DOMINANT) == "fp8k::gemm_tn_kernel<1, 0, false, 0, true, false, true>"
    assert bench.half_tile_kernel(bench.GEMM_KERNEL["fwd"]) == "fp8k::gemm_tn_kernel<0, 0, false, 0, true, false, false>"


def test_tail_rule_on_the_7b_layer():
    """256 CUs: the gate/up forward (1376 tiles) and the gate/up and down backward
    pairs (1632 and 1376 tiles) end in 96 tiles, run as half tiles; the other calls
    fill whole rounds (qkv 768, o 256, down forward 256; backward pairs 1024, 512)."""
    cfg = workloads.CONFIGS["layer7b"]
    M = cfg.M
    fwd, bwd = {}, {}
    for L in cfg.linears:
        fwd[L.name] = bench.tail_launch([(M, L.N, L.K, 0)], True, 256)
        bwd[L.name] = bench.tail_launch([(M, L.K, L.N, 0), (L.N, L.K, M, 0)], True, 256)
    assert fwd == {"qkv": False, "o": False, "gate_up": True, "down": False}
    assert bwd == {"qkv": False, "o": False, "gate_up": True, "down": True}
    # untransposed (MN-major) operands and matrices narrower than a tile never split
    assert not bench.tail_launch([(M, 22016, 4096, 0)], False, 256)
    assert not bench.tail_launch([(128, 22016, 4096, 0)], True, 256)


def test_traffic_summary_is_tied_to_the_gemm_source(monkeypatch):
    line = next(l for l in open(bench.TRAFFIC_SUMMARY) if l.startswith("TRAFFIC_JSON "))
    data = json.loads(line[len("TRAFFIC_JSON "):])
    per = data["per_dispatch_bytes"]
    if bench.gemm_code_hash() == data["gemm_code_sha256_16"]:
        want = int(per[DOMINANT] + 0.5 * per[bench.half_tile_kernel(DOMINANT)])
        assert bench.measured_traffic(DOMINANT, 0.5) == want
    monkeypatch.setattr(bench, "gemm_code_hash", lambda: "0" * 16)
    assert bench.measured_traffic(DOMINANT, 0.5) is None


def test_step_flop_count():
    """2 M N K per product, three products (forward, dgrad, wgrad) per linear."""
    for name, want in (("layer7b", 4.9736e12), ("layer14b", 13.529e12)):
        cfg = workloads.CONFIGS[name]
        flop = sum(6.0 * cfg.M * L.N * L.K for L in cfg.linears)
        assert flop == pytest.approx(want, rel=1e-4)
