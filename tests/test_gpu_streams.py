"""Concurrent use from several host threads, each on its own HIP stream.

The library keeps per-device state on the host (CU counts, the SwiGLU table's
device address) behind locks and its last error per thread.  Four threads each
run a chain of calls -- statistics, quantisation with transposed copies, the
forward GEMM, the paired backward GEMMs, the SwiGLU requant -- on their own
inputs and stream, many times over, while the others do the same; every
result must equal, byte for byte, the one the same chain gives alone on the
default stream, and an invalid call on one thread must leave the other
threads' error text untouched.
"""
import threading

import pytest
import torch

from gpu_util import E4M3, E5M2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def make_inputs(seed, M=512, K=768, N=1024, F=512):
    g = torch.Generator(device="cpu").manual_seed(seed)
    bf = lambda *s, sd=1.0: (torch.randn(s, generator=g) * sd).to(torch.bfloat16).cuda()
    return {"x": bf(M, K), "w": bf(N, K, sd=0.02), "dy": bf(M, N, sd=1e-3), "gu": bf(M, 2 * F, sd=2.0)}


def chain(fp8, t):
    """One pass of the calls; returns every output (device tensors)."""
    am = torch.zeros(3, dtype=torch.float32, device="cuda")
    fp8.absmax_accumulate_many([t["x"], t["w"]], [am[0:1], am[1:2]])
    qs, qts, _, invs = fp8.quantize_many([t["x"], t["w"]], E4M3, [am[0:1], am[1:2]], want_q=True, want_qt=True)
    y = fp8.gemm_fwd(qs[0], qs[1], invs[0], invs[1])
    ady = fp8.absmax(t["dy"])
    dyq, dyqt, _, idy = fp8.quantize(t["dy"], E5M2, ady, want_q=True, want_qt=True)
    dx, dw = fp8.gemm_backward(dyq, dyqt, E5M2, qts[1], qts[0], idy, invs[1], invs[0])
    hq, hqt, amh, ih = fp8.swiglu_requant(t["gu"], am[2:3], True, want_hq=True, want_hqt=True, accumulate=True)
    return [am, qs[0], qs[1], qts[0], qts[1], y, dyq, dyqt, dx, dw, hq, hqt, ih]


def test_threads_on_their_own_streams(fp8):
    n_threads, reps = 4, 20
    inputs = [make_inputs(100 + i) for i in range(n_threads)]
    say("streams: reference chains")
    ref = []
    for t in inputs:
        out = chain(fp8, t)
        torch.cuda.synchronize()
        ref.append([o.clone() for o in out])
    errors, results = [], [None] * n_threads

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(reps):
                    out = chain(fp8, inputs[i])
                s.synchronize()
                results[i] = [o.clone() for o in out]
                s.synchronize()
        except Exception as e:          # reported below, on the main thread
            errors.append((i, repr(e)))

    say("streams: threads", n_threads, "reps", reps)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=300)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(n_threads):
        for k, (a, b) in enumerate(zip(results[i], ref[i])):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a,
                               b.view(torch.uint8) if b.dtype != torch.float32 else b), (i, k)


def test_error_text_is_per_thread(fp8):
    """A refused call on one thread sets that thread's last error only."""
    lib = fp8._lib._lib
    seen = {}

    def bad():
        assert lib.fp8_absmax(None, 16, None, None) != 0
        seen["bad"] = lib.fp8_last_error().decode()

    th = threading.Thread(target=bad)
    th.start()
    th.join()
    # the main thread's text is whatever its own last call left: a good call clears it
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    fp8.absmax(x)
    torch.cuda.synchronize()
    assert seen["bad"].startswith("fp8_absmax"), seen
    assert lib.fp8_last_error().decode() == ""
