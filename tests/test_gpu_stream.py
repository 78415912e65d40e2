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
