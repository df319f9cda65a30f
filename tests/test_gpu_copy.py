"""The streaming-copy reference (fp8_stream_copy) copies every byte and nothing
beyond: sizes of one 16-byte vector, of less than one grid's worth, of several
grid-stride rounds with a ragged last round, and of a 256 MiB buffer (the size
the bandwidth reference is measured on)."""
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 16 * (2 * 256 * 512 * 3 + 77), 256 << 20])
def test_stream_copy_every_byte(fp8, nbytes):
    say("stream copy", nbytes)
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000003)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    guard = 4096
    buf = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    fp8.stream_copy(src, buf[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(buf[:nbytes], src)
    assert bool((buf[nbytes:] == 0xA5).all()), "bytes past the end were written"


def test_stream_copy_rejects_bad_arguments(fp8):
    a = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fp8.stream_copy(a, torch.zeros(32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(fp8.Fp8Error):
        fp8.stream_copy(a[:40], torch.zeros(40, dtype=torch.uint8, device="cuda"))
    with pytest.raises(fp8.Fp8Error):
        fp8.stream_copy(a[8:40], a[32:64])
