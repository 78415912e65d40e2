"""GPU checks of the streaming reference kernels (the practical-ceiling
copy and read that bench.py times beside the reductions): the copy is
byte-exact, and the XOR of the read's per-workgroup words equals the XOR of
every 32-bit word of the input."""
import numpy as np
import pytest

from gpu_util import dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, (16 << 20) + 48])
def test_stream_copy_is_exact(nbytes):
    rng = np.random.default_rng(nbytes)
    x = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32).view(np.int32)
    xd = dev(x)
    y = torch.full_like(xd, -1)
    fr.fr_stream_copy(xd, y)
    assert np.array_equal(host(y), x)


@pytest.mark.parametrize("nbytes", [0, 16, 4096, 16 * 1000 + 16, (16 << 20) + 48])
def test_stream_read_xor(nbytes):
    rng = np.random.default_rng(nbytes + 1)
    x = rng.integers(0, 2**32, size=max(nbytes // 4, 4), dtype=np.uint32)[: nbytes // 4]
    xd = dev(x.view(np.int32)) if nbytes else torch.empty(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(fr.FR_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    fr.lib.fr_stream_read(fr._ptr(xd), nbytes, fr._ptr(sink), fr._stream(None))
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    want = np.bitwise_xor.reduce(x) if nbytes else np.uint32(0)
    assert int(got) == int(want)


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, (16 << 20) + 48])
def test_stream_write_fills(nbytes):
    """Every word is the pattern, and the guard words past the end keep theirs."""
    y = torch.full((nbytes // 4 + 4,), -1, dtype=torch.int32, device="cuda")
    fr.lib.fr_stream_write(fr._ptr(y), nbytes, 0x9E3779B9, fr._stream(None))
    got = host(y).view(np.uint32)
    assert (got[: nbytes // 4] == 0x9E3779B9).all()
    assert (got[nbytes // 4:] == 0xFFFFFFFF).all()


def test_stream_empty_launches_back_to_back():
    """Empty launches between two clock marks: each costs at least the
    counter's resolution and far less than a millisecond."""
    khz = fr.fr_device_clock_khz()
    marks = torch.zeros(2, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    fr.fr_device_clock(marks, 0)
    for _ in range(100):
        fr.fr_stream_empty()
    fr.fr_device_clock(marks, 1)
    t = host(marks)
    us = (int(t[1]) - int(t[0])) / khz * 1000.0
    assert 0 < us < 100_000, us


def test_device_clock_marks_bracket_stream_work():
    """Two clock marks around a 256 MiB copy: the counter runs at the rate
    fr_device_clock_khz reports, the marks are ordered, and their distance
    covers the copy (512 MiB moved: at least 67 us at 8 TB/s) without being
    absurd."""
    khz = fr.fr_device_clock_khz()
    assert 1000 <= khz <= 10_000_000
    marks = torch.zeros(2, dtype=torch.int64, device="cuda")
    x = torch.zeros((256 << 20) // 4, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    fr.fr_device_clock(marks, 0)
    fr.fr_stream_copy(x, y)
    fr.fr_device_clock(marks, 1)
    t = host(marks)
    us = (int(t[1]) - int(t[0])) / khz * 1000.0
    assert (256 << 21) / 8e6 <= us < 100_000, us
    with pytest.raises(ValueError):
        fr.fr_device_clock(marks, 2)


def test_pointer_chase_follows_the_chain():
    """The latency walk reaches the index a host walk of the same chain
    reaches; indices outside the array are taken as 0 (clamped), so the walk
    never leaves it."""
    rng = np.random.default_rng(5)
    n, stride = 1 << 14, 16
    pos = np.arange(0, n, stride)
    order = pos[rng.permutation(pos.size)]
    chain = np.zeros(n, dtype=np.int64)
    chain[order] = np.roll(order, -1)
    chain[order[7]] = n + 12345  # out of range: the walk goes to 0
    chain[0] = order[0]
    cd = dev(chain.astype(np.uint32).view(np.int32))
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    for steps in (0, 1, 5, 100, 3000):
        fr.fr_pointer_chase(cd, steps, int(order[0]), out)
        i = int(order[0])
        for _ in range(steps):
            nx = int(chain[i])
            i = nx if nx < n else 0
        got = host(out)
        assert int(got[1]) == i, steps
        assert int(got[0]) >= 0
