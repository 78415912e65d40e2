"""GPU parity: the pointwise kernels against the fp64 oracle ("Stax (4)", 9.3).

fr_add_2d: out = a + b where either operand may be a transposed view (Listing
9.2, Example 6.1: x.t() + y at 256 x 512). Bit-exact: every output is the
correctly rounded fp32 sum on both sides.

fr_gelu_backward: dx = dy * (Phi(h) + h phi(h)) (Listing 9.3, Example 5.1:
2048 elements, one broadcast upstream value). fp32 within 1e-5 * |dy| (Phi(h)
+ |h| phi(h)) + 1e-6 (the fp32 rule on the terms that form dx; the device's
erf carries an absolute error of a few 1e-8 where 1 + erf cancels); bf16
within one bf16 ulp of the oracle's rounded value, or that fp32 rule.
Inputs: h ~ N(0, 2^2) with +-0, +-inf and NaN planted, dy ~ N(0, 1).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_of, bf16_bits_tensor, bf16_to_f64, check_bf16, check_fp32, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402

# ------------------------------------------------------------------ 2-D add


def add_case(rows, cols, ta, tb, seed, pad=0):
    """Device operands of shape [rows, cols]: a transposed operand is the .t()
    of a [cols, rows (+pad)] array, a row-major one a [rows, cols (+pad)] view."""
    def operand(t, stream):
        if t:
            base = synth.normal((cols, rows + pad), seed, stream=stream)
            return base, dev(base)[:, :rows].t()
        base = synth.normal((rows, cols + pad), seed, stream=stream)
        return base, dev(base)[:, :cols]
    ha, da = operand(ta, 1)
    hb, db = operand(tb, 2)
    va = ha[:, :rows].T if ta else ha[:, :cols]
    vb = hb[:, :rows].T if tb else hb[:, :cols]
    return va, vb, da, db


def test_add_2d_example_6_1():
    # x is [512, 256]; out = x.t() + y with y [256, 512]
    x = synth.normal((512, 256), 61, stream=1)
    y = synth.normal((256, 512), 61, stream=2)
    xd, yd = dev(x), dev(y)
    out = torch.empty((256, 512), dtype=torch.float32, device="cuda")
    fr.fr_add_2d(xd.t(), yd, out)
    assert np.array_equal(host(out), oracle.add_2d(x.T, y))
    assert fr.fr_plan_query(fr.FR_OP_ADD_2D, 256, 512).grid == 16  # 64 x 128 tiles


SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (64, 64), (65, 63), (128, 200), (200, 130), (1000, 777), (257, 4100)]


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("shape", SHAPES)
def test_add_2d_layouts_and_ragged_tiles(shape, ta, tb):
    rows, cols = shape
    va, vb, da, db = add_case(rows, cols, ta, tb, seed=rows * 7 + cols)
    out = torch.full((rows, cols), -7.0, dtype=torch.float32, device="cuda")
    fr.fr_add_2d(da, db, out)
    assert np.array_equal(host(out), oracle.add_2d(va, vb)), (shape, ta, tb)


@pytest.mark.parametrize("ta,tb", [(True, False), (False, True), (True, True)])
def test_add_2d_padded_and_unaligned(ta, tb):
    # strides that are not multiples of 4 elements: element accesses throughout
    rows, cols = 150, 97
    va, vb, da, db = add_case(rows, cols, ta, tb, seed=5, pad=3)
    big = torch.full((rows, cols + 5), -7.0, dtype=torch.float32, device="cuda")
    out = big[:, 1:cols + 1]  # 4-byte aligned base, row stride 102
    fr.fr_add_2d(da, db, out)
    got = host(big)
    assert np.array_equal(got[:, 1:cols + 1], oracle.add_2d(va, vb))
    assert np.all(got[:, 0] == -7.0) and np.all(got[:, cols + 1:] == -7.0)  # nothing outside out


def test_add_2d_in_place_and_empty():
    rows, cols = 300, 260
    va, vb, da, db = add_case(rows, cols, True, False, seed=9)
    want = oracle.add_2d(va, vb)
    fr.fr_add_2d(da, db, db)  # out = b, same layout
    assert np.array_equal(host(db), want)
    e = torch.empty((0, 5), dtype=torch.float32, device="cuda")
    fr.fr_add_2d(e, e, e)
    with pytest.raises(ValueError):
        fr.fr_add_2d(da, db, da.t().contiguous().t())  # out column-major: the C ABI takes row-major only


def test_add_2d_rejects_other_layouts():
    x = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    out = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(fr.FrError) as ei:
        fr.fr_add_2d(x[::2, ::2], x[:32, :32], out)
    assert ei.value.status == fr.FR_E_STRIDE
    sq = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(fr.FrError) as ei:
        fr.fr_add_2d(sq.t(), x, sq)  # out aliases a transposed operand
    assert ei.value.status == fr.FR_E_ARG


def test_add_2d_full_size_sampled():
    # 8192 x 8192 with the first operand transposed, the launch the benchmark times
    n = 8192
    x = synth.normal((n, n), 62, stream=1)
    y = synth.normal((n, n), 62, stream=2)
    xd, yd = dev(x), dev(y)
    out = torch.empty((n, n), dtype=torch.float32, device="cuda")
    fr.fr_add_2d(xd.t(), yd, out)
    got = host(out)
    rng = np.random.default_rng(3)
    ri = np.sort(rng.choice(n, 96, replace=False))
    ci = np.sort(rng.choice(n, 96, replace=False))
    want = oracle.add_2d(np.ascontiguousarray(x.T[np.ix_(ri, ci)]), np.ascontiguousarray(y[np.ix_(ri, ci)]))
    assert np.array_equal(got[np.ix_(ri, ci)], want)
    # every row and column: the row sums agree with the exact sums of the inputs
    assert np.allclose(got.sum(axis=1, dtype=np.float64), x.sum(axis=0, dtype=np.float64) +
                       y.sum(axis=1, dtype=np.float64), rtol=0, atol=1e-3)


# ------------------------------------------------------------ GELU backward


def gelu_inputs(n, seed, plant=True):
    h = synth.normal((n,), seed, stream=3, std=2.0)
    if plant and n >= 8:
        h[:6] = [0.0, -0.0, np.inf, -np.inf, np.nan, -0.7518]
    dy = synth.normal((n,), seed, stream=4)
    return h, dy


def run_gelu(h, dy, bf16=False, offset=0, inplace=False):
    """Device call; offset > 0 shifts every array by that many elements
    (unaligned bases: element accesses)."""
    n = h.size
    if bf16:
        hb, gb = synth.to_bf16(h), synth.to_bf16(dy)
        hd = bf16_bits_tensor(np.concatenate([np.zeros(offset, np.uint16), hb]))[offset:]
        gd = bf16_bits_tensor(np.concatenate([np.zeros(offset, np.uint16), gb]))[offset:]
        xd = torch.empty(n + offset, dtype=torch.bfloat16, device="cuda")[offset:]
    else:
        hd = dev(np.concatenate([np.zeros(offset, np.float32), h]))[offset:]
        gd = dev(np.concatenate([np.zeros(offset, np.float32), dy]))[offset:]
        xd = torch.empty(n + offset, dtype=torch.float32, device="cuda")[offset:]
    if inplace:
        xd = hd
    fr.fr_gelu_backward(gd, hd, xd)
    return bf16_bits_of(xd) if bf16 else host(xd)


def check_gelu(got, h, dy, bf16, what):
    if bf16:
        h64, g64 = bf16_to_f64(synth.to_bf16(h)), bf16_to_f64(synth.to_bf16(dy))
        dx64, mag = oracle.gelu_backward(g64, h64)
        check_bf16(got, oracle.round_bf16(dx64), dx64, mag, what=what)
    else:
        dx64, mag = oracle.gelu_backward(dy.astype(np.float64), h.astype(np.float64))
        check_fp32(got, dx64, terms=mag, what=what)


def test_gelu_backward_example_5_1():
    # 2048 elements, the upstream gradient of a scalar loss broadcast
    h, _ = gelu_inputs(2048, 51)
    dy = np.array([0.75], dtype=np.float32)
    got = run_gelu(h, dy)
    dx64, mag = oracle.gelu_backward(0.75, h.astype(np.float64))
    check_fp32(got, dx64, terms=mag, what="example 5.1")
    assert got[0] == 0.375 and np.isnan(got[2]) and np.isnan(got[3]) and np.isnan(got[4])


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("bcast", [False, True])
@pytest.mark.parametrize("n", [1, 3, 8, 9, 1000, 2048, 65537, (1 << 20) + 5])
def test_gelu_backward_sizes(n, bcast, bf16):
    h, dy = gelu_inputs(n, 52 + n)
    if bcast:
        dy = dy[:1].copy()
    got = run_gelu(h, dy, bf16=bf16)
    check_gelu(got, h, dy, bf16, what=f"n={n} bcast={bcast} bf16={bf16}")


@pytest.mark.parametrize("bf16", [False, True])
def test_gelu_backward_unaligned_and_in_place(bf16):
    n = 70001
    h, dy = gelu_inputs(n, 53)
    check_gelu(run_gelu(h, dy, bf16=bf16, offset=1), h, dy, bf16, what="unaligned")
    check_gelu(run_gelu(h, dy, bf16=bf16, inplace=True), h, dy, bf16, what="in place")


def test_gelu_backward_full_size_sampled():
    # 2^28 fp32 elements, one broadcast upstream value: the benchmark's launch
    n = 1 << 28
    h = synth.normal((n,), 54, stream=3, std=2.0)
    hd = dev(h)
    dy = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    dx = torch.empty_like(hd)
    fr.fr_gelu_backward(dy, hd, dx)
    idx = np.random.default_rng(5).choice(n, 1 << 16, replace=False)
    idx = np.concatenate([idx, np.arange(n - 37, n)])  # the last vectors and the tail
    got = dx[torch.from_numpy(idx).cuda()].cpu().numpy()
    dx64, mag = oracle.gelu_backward(0.5, h[idx].astype(np.float64))
    check_fp32(got, dx64, terms=mag, what="2^28 sampled")
    del hd, dx


def test_gelu_backward_argument_errors():
    h = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fr.fr_gelu_backward(torch.zeros(3, device="cuda"), h, h)
    with pytest.raises(ValueError):
        fr.fr_gelu_backward(h, h, h.to(torch.bfloat16))
