"""GPU: recorded regions ("Stax (4)", 9.9) replay what they recorded.

A region records the example 1.1 sums (64 x 128, the tiny shape whose time
is launch overhead) and a small softmax on a side stream, then is replayed
several times with new input values copied into the recorded buffers and
eager work in between; every replay must match the fp64 oracle on the
values it was given (the shared tolerance rule) and equal an eager run bit
for bit (the same kernels on the same inputs). A different key runs directly and
keeps the recording; the legacy default stream cannot be captured and sends
the region to its fallback state, where results stay correct.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_fp32, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


def buffers(seed):
    a, b, _ = synth.sum_relu_add_inputs(64, 128, seed=seed)
    x = synth.softmax_inputs(32, 1000, seed=seed)
    return {"a": dev(a), "b": dev(b), "x": dev(x),
            "out": torch.empty(64, dtype=torch.float32, device="cuda"),
            "y": torch.empty((32, 1000), dtype=torch.float32, device="cuda")}


def region_fn(buf):
    def fn(stream):
        fr.fr_sum_relu_add(buf["a"], buf["b"], buf["out"], stream=stream)
        fr.fr_softmax_rows(buf["x"], buf["y"], stream=stream)
    return fn


def key_of(buf):
    return [buf[k].data_ptr() for k in ("a", "b", "x", "out", "y")] + [64, 128, 32, 1000]


def eager(buf):
    out = torch.empty_like(buf["out"])
    y = torch.empty_like(buf["y"])
    fr.fr_sum_relu_add(buf["a"], buf["b"], out)
    fr.fr_softmax_rows(buf["x"], y)
    torch.cuda.synchronize()
    return host(out), host(y)


def check_oracle(buf, what):
    """The region's outputs against the oracle on the inputs it read."""
    _, ref = oracle.sum_relu_add(host(buf["a"]), host(buf["b"]))
    check_fp32(host(buf["out"]), ref, what=f"{what}: sum_relu_add")
    y64, _ = oracle.softmax_rows(host(buf["x"]))
    check_fp32(host(buf["y"]), y64, what=f"{what}: softmax")


def test_region_records_then_replays_new_values():
    buf = buffers(1001)
    side = torch.cuda.Stream()
    region = fr.Region()
    with torch.cuda.stream(side):
        region.run(key_of(buf), region_fn(buf))
    side.synchronize()
    assert region.state == fr.FR_REGION_RECORDED and region.counts() == (1, 0)
    check_oracle(buf, "recording run")
    want = eager(buf)
    assert np.array_equal(host(buf["out"]), want[0]) and np.array_equal(host(buf["y"]), want[1])
    for rep in range(4):
        nb = buffers(2000 + rep)
        for k in ("a", "b", "x"):  # new values at the recorded addresses
            buf[k].copy_(nb[k])
        torch.cuda.synchronize()
        _ = (buf["a"] * 2).sum().item()  # eager work between replays
        with torch.cuda.stream(side):
            region.run(key_of(buf), region_fn(buf))
        side.synchronize()
        check_oracle(buf, f"replay {rep}")
        want = eager(buf)
        assert np.array_equal(host(buf["out"]), want[0]), rep
        assert np.array_equal(host(buf["y"]), want[1]), rep
    assert region.counts() == (5, 0)


def test_region_other_key_runs_directly():
    buf, other = buffers(3001), buffers(3002)
    side = torch.cuda.Stream()
    region = fr.Region()
    with torch.cuda.stream(side):
        region.run(key_of(buf), region_fn(buf))
        region.run(key_of(other), region_fn(other))  # other addresses: direct
        region.run(key_of(buf), region_fn(buf))      # recorded key again: replay
    side.synchronize()
    assert region.state == fr.FR_REGION_RECORDED and region.counts() == (2, 1)
    check_oracle(buf, "replay after a direct run")
    check_oracle(other, "direct run")
    want = eager(other)
    assert np.array_equal(host(other["out"]), want[0]) and np.array_equal(host(other["y"]), want[1])


def test_region_fallback_on_the_default_stream_and_on_errors():
    buf = buffers(4001)
    region = fr.Region()
    region.run(key_of(buf), region_fn(buf), stream=0)  # legacy default stream: cannot be captured
    torch.cuda.synchronize()
    assert region.state == fr.FR_REGION_FALLBACK and region.counts() == (0, 1)
    check_oracle(buf, "fallback run")
    want = eager(buf)
    assert np.array_equal(host(buf["out"]), want[0])
    bad = fr.Region()
    side = torch.cuda.Stream()

    def failing(stream):
        fr.fr_sum_relu_add(buf["a"], buf["b"], buf["out"], stream=stream)
        fr.fr_softmax_rows(buf["x"], buf["y"][:, :999], stream=stream)  # shape mismatch: the wrapper raises

    with torch.cuda.stream(side):
        with pytest.raises(ValueError):
            bad.run(key_of(buf), failing)
    side.synchronize()
    assert bad.state == fr.FR_REGION_FALLBACK
