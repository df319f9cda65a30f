"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between replays,
reproduces the eager step's bytes exactly.

The step: clear a statistics buffer (a fill kernel), X and W statistics in one
launch, their e4m3 quantisation with transposed copies in one launch, the forward GEMM, the
gate/up GEMM with the SwiGLU statistic in its epilogue and the requant that
uses it, e5m2 quantisation of dY, the paired backward GEMMs, and the SwiGLU
backward.

A second test records a fresh process's very first SwiGLU calls (the SwiGLU
tables are constant data of the library, so nothing has to run before a
capture) and checks its replays against eager calls made afterwards.
"""
import os
import subprocess
import sys

import pytest
import torch

from gpu_util import E4M3, E5M2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def test_step_replays_in_a_graph(fp8):
    M, K, N, F = 512, 1024, 768, 1024
    g = torch.Generator(device="cpu").manual_seed(21)
    bf = lambda *s, sd=1.0: (torch.randn(s, generator=g) * sd).to(torch.bfloat16).cuda()
    x, w, dy = bf(M, K), bf(N, K, sd=0.02), bf(M, N, sd=1e-3)
    w_gu, dh = bf(2 * F, K, sd=0.02), bf(M, F, sd=1e-3)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda: torch.empty(1, dtype=torch.float32, device="cuda")
    stats = torch.empty(8, dtype=torch.float32, device="cuda")
    out = {
        "xq": u8(M, K), "xqt": u8(K, M), "wq": u8(N, K), "wqt": u8(K, N), "guq": u8(2 * F, K),
        "dyq": u8(M, N), "dyqt": u8(N, M), "hq": u8(M, F), "hqt": u8(F, M), "dgq": u8(M, 2 * F),
        "dgqt": u8(2 * F, M),
        "y": torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
        "gu": torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda"),
        "dx": torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
        "dw": torch.empty((N, K), dtype=torch.bfloat16, device="cuda"),
        "ix": f32(), "iw": f32(), "igu": f32(), "idy": f32(), "ih": f32(), "idg": f32(), "dg_am": f32(),
        "stats": stats,
    }
    o = out

    def step():
        stats.zero_()
        fp8.absmax_accumulate_many([x, w, w_gu], [stats[0:1], stats[1:2], stats[2:3]])
        fp8.quantize_many([x, w], E4M3, [stats[0:1], stats[1:2]], want_qt=True, qs=[o["xq"], o["wq"]],
                          qts=[o["xqt"], o["wqt"]], inv_scales=[o["ix"], o["iw"]])
        fp8.quantize(w_gu, E4M3, stats[2:3], q=o["guq"], inv_scale=o["igu"])
        fp8.gemm_fwd(o["xq"], o["wq"], o["ix"], o["iw"], out=o["y"])
        fp8.gemm_fwd_swiglu_absmax(o["xq"], o["guq"], o["ix"], o["igu"], stats[3:4], out=o["gu"])
        fp8.swiglu_requant(o["gu"], stats[3:4], False, hq=o["hq"], hqt=o["hqt"], inv_scale_h=o["ih"])
        fp8.absmax(dy, stats[4:5], accumulate=True)
        fp8.quantize(dy, E5M2, stats[4:5], q=o["dyq"], qt=o["dyqt"], inv_scale=o["idy"])
        fp8.gemm_backward(o["dyq"], o["dyqt"], E5M2, o["wqt"], o["xqt"], o["idy"], o["iw"], o["ix"],
                          dx=o["dx"], dw=o["dw"])
        fp8.swiglu_backward(o["gu"], dh, E5M2, absmax=o["dg_am"], q=o["dgq"], qt=o["dgqt"], inv_scale=o["idg"])

    say("graph: eager step")
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    graph = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = bf(4096, 512)
    for rep in range(4):
        say("graph: replay", rep)
        for v in out.values():                # garbage between replays, and unrelated eager work
            if v.dtype == torch.uint8:
                v.fill_(0x5A)
            else:
                v.fill_(float("nan"))
        fp8.absmax(other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v.view(torch.uint8), ref[k].view(torch.uint8)), f"replay {rep}: {k} differs"


FIRST_CALLS_CAPTURED = r"""
import sys, torch
import fp8_precision_amd as fp8
M, K, F = 256, 512, 512
g = torch.Generator().manual_seed(5)
gu = (torch.randn(M, 2 * F, generator=g) * 3).to(torch.bfloat16).cuda()
xq = (torch.randn(M, K, generator=g)).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
wq = (torch.randn(2 * F, K, generator=g) * 0.5).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
one = torch.ones(1, dtype=torch.float32, device="cuda")
outs = lambda: dict(am=torch.zeros(1, dtype=torch.float32, device="cuda"),
                    hq=torch.empty(M, F, dtype=torch.uint8, device="cuda"),
                    hqt=torch.empty(F, M, dtype=torch.uint8, device="cuda"),
                    inv=torch.empty(1, dtype=torch.float32, device="cuda"),
                    am2=torch.zeros(1, dtype=torch.float32, device="cuda"),
                    y=torch.empty(M, 2 * F, dtype=torch.bfloat16, device="cuda"))
def step(o):
    o["am"].zero_()
    o["am2"].zero_()
    fp8.swiglu_requant(gu, absmax_h=o["am"], want_hqt=True, hq=o["hq"], hqt=o["hqt"], inv_scale_h=o["inv"],
                       accumulate=True)
    fp8.gemm_fwd_swiglu_absmax(xq, wq, one, one, o["am2"], out=o["y"])
torch.cuda.synchronize()
cap = outs()
graph = torch.cuda.CUDAGraph()
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(side):
    with torch.cuda.graph(graph, stream=side):
        step(cap)          # the process's first SwiGLU and gate/up-statistic calls
torch.cuda.current_stream().wait_stream(side)
torch.cuda.synchronize()
ref = outs()
step(ref)
torch.cuda.synchronize()
for r in range(3):
    for t in cap.values():
        t.fill_(0)
    graph.replay()
    torch.cuda.synchronize()
    for k in cap:
        if not torch.equal(cap[k].view(torch.uint8), ref[k].view(torch.uint8)):
            print(f"replay {r}: {k} differs from the eager call"); sys.exit(1)
print("first calls captured: 3 replays bit-exact")
"""


def test_first_swiglu_calls_of_a_process_capture():
    say("fresh process: first SwiGLU calls under capture")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", FIRST_CALLS_CAPTURED], cwd=root, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-exact" in r.stdout
