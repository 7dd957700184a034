"""The plain streams of known bytes (synth: copy, read, write) that calibrate
the memory counters and give the rate a plain stream reaches: each moves
exactly the bytes it is charged with, ragged tails included."""
import pytest

import synth

from _helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("n", [1, 3, 4, 2047, 2048, 2049, 4096 * 3 + 5, 1 << 22])
def test_streams_move_exactly_their_elements(n):
    say(f"case streams n={n}")
    pad = 64
    src = torch.randn(n + 2 * pad, device="cuda")
    dst = torch.full((n + 2 * pad,), -7.0, device="cuda")
    sink = torch.zeros(256, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    # 16-byte aligned starting points inside the padded buffers
    synth.stream_copy(src[pad:].data_ptr(), dst[pad:].data_ptr(), n, s)
    synth.stream_read(src[pad:].data_ptr(), n, sink.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(dst[pad:pad + n], src[pad:pad + n])
    assert bool((dst[:pad] == -7.0).all()) and bool((dst[pad + n:] == -7.0).all())
    assert bool((sink == 0).all())
    synth.stream_write(dst[pad:].data_ptr(), n, 2.5, s)
    torch.cuda.synchronize()
    assert bool((dst[pad:pad + n] == 2.5).all())
    assert bool((dst[:pad] == -7.0).all()) and bool((dst[pad + n:] == -7.0).all())


def test_streams_reject_misaligned_pointers():
    a = torch.zeros(64, device="cuda")
    with pytest.raises(RuntimeError):
        synth.stream_copy(a.data_ptr() + 4, a.data_ptr(), 8)
    with pytest.raises(RuntimeError):
        synth.stream_write(a.data_ptr() + 4, 8, 1.0)
