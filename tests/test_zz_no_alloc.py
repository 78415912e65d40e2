"""GPU: fr_sumsq_full_noalloc, the sum of squares whose split partials live
in the library's own device array, called through the C ABI.

It must give exactly the bits of fr_sumsq_full (same kernels, same
partition) with a caller workspace, on two calls in a row, the second with
a smaller input (the array keeps the first call's partials, which must not
leak into the second), and match the fp64 oracle within
|s - ref| <= 1e-5 * ref + 1e-6 (every term is nonnegative)."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


def with_workspace(xd):
    n = xd.numel()
    ws = torch.empty(max(fr.fr_sumsq_full_workspace_bytes(n), 16) // 4, dtype=torch.float32, device="cuda")
    out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    fr.fr_sumsq_full(xd, out, ws=ws)
    return host(out).view(np.uint32)[0]


def no_alloc(xd):
    out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    st = fr.lib.fr_sumsq_full_noalloc(fr._ptr(xd), xd.numel(), fr._ptr(out), fr.FR_F32, fr._stream(None))
    assert st == fr.FR_OK, fr.lib.fr_status_string(st)
    return host(out).view(np.uint32)[0]


def test_no_alloc_sumsq_matches_workspace_form_twice():
    for n, seed in ((1 << 28, 4201), ((1 << 20) + 12345, 4202), (5000, 4203)):
        x = synth.sumsq_inputs(n, seed=seed)
        xd = dev(x)
        got = no_alloc(xd)
        want = with_workspace(xd)
        assert got == want, f"n={n}: bits {got:#x} against {want:#x}"
        ref = oracle.sumsq(x)
        val = float(np.array([got], dtype=np.uint32).view(np.float32)[0])
        assert abs(val - ref) <= 1e-5 * ref + 1e-6, (n, val, ref)


def test_no_alloc_sumsq_edges():
    # n = 0 is the empty sum; one element; a non-split length; x = 1 is exact
    for n in (0, 1, 2048, 98432):
        xd = torch.ones(max(n, 1), dtype=torch.float32, device="cuda")[:n]
        out = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        st = fr.lib.fr_sumsq_full_noalloc(fr._ptr(xd) if n else None, n, fr._ptr(out), fr.FR_F32,
                                         fr._stream(None))
        assert st == fr.FR_OK
        assert float(host(out)[0]) == float(n)
    # beyond the largest size: refused before anything runs
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    xd = torch.ones(4, dtype=torch.float32, device="cuda")
    assert fr.lib.fr_sumsq_full_noalloc(fr._ptr(xd), 1 << 30, fr._ptr(out), fr.FR_F32, None) == fr.FR_E_SIZE
    assert fr.lib.fr_sumsq_full_noalloc(fr._ptr(xd), 4, fr._ptr(out), fr.FR_BF16, None) == fr.FR_E_DTYPE
    assert fr.lib.fr_sumsq_full_noalloc(fr._ptr(xd), 4, None, fr.FR_F32, None) == fr.FR_E_NULL
