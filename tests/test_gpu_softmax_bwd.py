"""GPU parity: fr_softmax_rows_backward against the fp64 oracle.

dx = y (dy - sum_k dy_k y_k) per row (the derivative of the row softmax of
"Stax (4)", 9.5). y is the oracle's forward output on the pages' softmax
inputs, rounded to fp32 (both sides get the same y), dy ~ N(0, 1). Tolerance per element: |dx - dx_ref| <=
1e-5 * (|y_j dy_j| + y_j sum_k |dy_k y_k|) + 1e-6. Ragged rows: the tails of
y and dy hold NaN and must not be read; the tail of dx must stay untouched.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_fp32, dev, forced, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402

FORMS = {"auto": fr.FR_FORM_AUTO, "per": fr.FR_FORM_PER, "red": fr.FR_FORM_RED}


def inputs(rows, cols, seed, lengths=None):
    x = synth.softmax_inputs(rows, cols, seed=seed)
    y_h = oracle.softmax_rows(x)[0].astype(np.float32)
    dy = synth.normal((rows, cols), seed, stream=7)
    if lengths is not None:
        for r, n in enumerate(lengths):
            y_h[r, max(n, 0):] = np.nan
            dy[r, max(n, 0):] = np.nan
    return y_h, dy


def run(y, dy, lengths=None, form="auto", inplace=False):
    yd, dyd = dev(y), dev(dy)
    dx = dyd if inplace else torch.full_like(yd, -3.0)
    L = None if lengths is None else dev(np.asarray(lengths, dtype=np.int32))
    with forced(FORMS[form]):
        fr.fr_softmax_rows_backward(yd, dyd, dx, lengths=L)
    return host(dx)


def compare(y, dy, got, lengths=None, what=""):
    dx64, mag = oracle.softmax_backward_rows(y, dy, lengths=lengths)
    valid = ~np.isnan(dx64)
    check_fp32(np.where(valid, got, 0.0), np.where(valid, dx64, 0.0), terms=np.where(valid, mag, 0.0), what=what)


def test_softmax_backward_4096x1024():
    y, dy = inputs(4096, 1024, seed=2001)
    got = run(y, dy)
    compare(y, dy, got, what="4096x1024")
    assert np.allclose(got.sum(axis=1), 0.0, atol=1e-5)  # sum_j dx_j = s (1 - sum_j y_j) ~ 0


SHAPES = [(1, 1), (7, 13), (33, 31), (65, 33), (256, 1000), (3, 1024), (5, 2048), (2, 2049), (4, 20000),
          (2, 70001)]


@pytest.mark.parametrize("form", ["per", "red"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_softmax_backward_forms(form, shape):
    rows, cols = shape
    y, dy = inputs(rows, cols, seed=2500 + rows + cols)
    if form == "per" and cols > 2048:
        # rows longer than the persistent capacity: the forced call is refused
        with pytest.raises(fr.FrError) as e:
            run(y, dy, form=form)
        assert e.value.status == fr.FR_E_ARG
        return
    got = run(y, dy, form=form)
    compare(y, dy, got, what=f"{form} {rows}x{cols}")


@pytest.mark.parametrize("cols", [1000, 2048, 50257])
def test_softmax_backward_ragged_rows(cols):
    rows = 12
    L = np.array([0, 1, 3, 4, 5, cols - 1, cols, cols + 9, 17, 2, cols // 2, 7], dtype=np.int32)
    y, dy = inputs(rows, cols, seed=2600 + cols, lengths=np.clip(L, 0, cols))
    got = run(y, dy, lengths=L)
    compare(y, dy, got, lengths=L, what=f"ragged {cols}")
    for r, n in enumerate(np.clip(L, 0, cols)):
        assert np.all(got[r, n:] == -3.0), f"row {r}: the tail was written"


def test_softmax_backward_in_place_and_strides():
    y, dy = inputs(40, 700, seed=2700)
    got = run(y, dy, inplace=True)
    compare(y, dy, got, what="dx = dy")
    # row strides: views into wider buffers
    yw = np.full((40, 768), np.nan, dtype=np.float32)
    gw = np.full((40, 768), np.nan, dtype=np.float32)
    yw[:, :700], gw[:, :700] = y, dy
    yd, gd = dev(yw), dev(gw)
    out = torch.full((40, 800), -3.0, dtype=torch.float32, device="cuda")
    fr.fr_softmax_rows_backward(yd[:, :700], gd[:, :700], out[:, :700])
    o = host(out)
    compare(y, dy, np.ascontiguousarray(o[:, :700]), what="strided")
    assert np.all(o[:, 700:] == -3.0)


def test_softmax_backward_is_deterministic():
    y, dy = inputs(64, 30000, seed=2800)
    outs = [run(y, dy) for _ in range(3)]
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])
