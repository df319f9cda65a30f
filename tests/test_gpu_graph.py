"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between replays,
reproduces the eager step's bytes exactly.

The step: clear a statistics buffer (a fill kernel), X and W statistics in one
launch, e4m3 quantisation with transposed copies, the forward GEMM, the
gate/up GEMM with the SwiGLU statistic in its epilogue and the requant that
uses it, e5m2 quantisation of dY, the paired backward GEMMs, and the SwiGLU
backward.  The first SwiGLU call on the device (which builds its tables and
waits for them once) runs before the capture.
"""
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
        fp8.quantize(x, E4M3, stats[0:1], q=o["xq"], qt=o["xqt"], inv_scale=o["ix"])
        fp8.quantize(w, E4M3, stats[1:2], q=o["wq"], qt=o["wqt"], inv_scale=o["iw"])
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
