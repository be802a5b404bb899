"""GPU check of the measurement-control copy the benchmark times beside the
update (page "Composing multi-kernel blocks in Python", section "Measuring a
block honestly": a plain baseline in the same run).  It must copy exactly the
bytes it is given, ragged sizes included, and touch nothing past them."""
import pytest
import torch

import depthwise_causal_conv1d_amd as dc

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.mark.parametrize("nbytes", [16, 1008, 16384, 16400, 16 * 1000 * 1000 + 48, 33_619_968 // 2])
def test_stream_copy_copies_exactly(nbytes):
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(dev)
    buf = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=dev)
    dst = buf[GUARD:GUARD + nbytes]
    dc.stream_copy(dst, src)
    torch.cuda.synchronize()
    assert dc.dcconv_last_kernel() == "stream_copy_v8"
    assert torch.equal(dst, src)
    assert bool((buf[:GUARD] == 0xA5).all()) and bool((buf[GUARD + nbytes:] == 0xA5).all())


@pytest.mark.parametrize("us", [50.0, 400.0])
def test_busy_spin_lasts_about_as_asked(us):
    """The benchmark's head: it must hold the stream for about the time asked
    (wall-clock bound, whatever the shader clock) and then end."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dc.busy_spin(1.0)  # first launch out of the timing
    a.record(stream)
    dc.busy_spin(us)
    b.record(stream)
    torch.cuda.synchronize()
    assert dc.dcconv_last_kernel() == "busy_spin"
    took = a.elapsed_time(b) * 1e3
    assert 0.9 * us <= took <= us + 200.0, took
