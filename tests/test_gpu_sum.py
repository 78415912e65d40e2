"""GPU parity: fr_sum_relu_add (Example 1.1), fr_sumsq_rows and
fr_sumsq_full against the fp64 oracle.

Tolerance: |out - ref| <= 1e-5 * sum|terms| + 1e-6; every term is
nonnegative, so sum|terms| is the reference itself. Bit-exact pins: inputs
on a coarse grid (every partial sum exact in fp32), x = 1 (exact integer
sums), and run-to-run identity of the split full reduction.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_fp32, dev, forced, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402

FORMS = {"per": fr.FR_FORM_PER, "red": fr.FR_FORM_RED, "split": fr.FR_FORM_SPLIT}


def ws_for(rows, cols):
    n = fr.fr_sum_workspace_bytes(rows, cols)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")


def gpu_sum_relu_add(a, b, form=fr.FR_FORM_AUTO, ws=True, out_stride=1):
    rows, cols = a.shape
    out = torch.full((rows * out_stride,), -1.0, dtype=torch.float32, device="cuda")
    o = out[::out_stride]
    with forced(form):
        fr.fr_sum_relu_add(dev(a), dev(b), o, ws=ws_for(rows, cols) if ws else None)
    return host(out)[::out_stride]


# ------------------------------------------------------------------ Example 1.1


@pytest.mark.parametrize("seed", [1001, 1003, 1005])
def test_example_1_1_64x128(seed):
    a, b, _ = synth.sum_relu_add_inputs(64, 128, seed=seed)
    out = gpu_sum_relu_add(a, b)
    _, ref = oracle.sum_relu_add(a, b)
    check_fp32(out, ref, what=f"Example 1.1 seed {seed}")
    assert abs(ref.mean() - 128 * 2 / 3) < 5  # E[2 relu(a+b)] = 2/3 per element (sanity)


def test_example_1_1_nan_rows():
    a, b, nan_rows = synth.sum_relu_add_inputs(64, 128, seed=1002, n_nan=4)
    for form in ("per", "red", "split"):
        out = gpu_sum_relu_add(a, b, form=FORMS[form])
        assert set(np.nonzero(np.isnan(out))[0].tolist()) == set(nan_rows.tolist()), form
        _, ref = oracle.sum_relu_add(a, b)
        check_fp32(out, ref, what=f"NaN variant {form}")


@pytest.mark.parametrize("form", ["per", "red", "split"])
def test_exact_grid_is_bit_exact(form):
    rng = np.random.default_rng(77)
    grid = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32)
    for rows, cols in [(64, 128), (7, 13), (33, 2048), (3, 9000)]:
        if form == "per" and cols > 2048:
            continue
        a = grid[rng.integers(0, 5, size=(rows, cols))]
        b = grid[rng.integers(0, 5, size=(rows, cols))]
        out = gpu_sum_relu_add(a, b, form=FORMS[form])
        ref, _ = oracle.sum_relu_add(a, b)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), f"{form} {rows}x{cols}"


SHAPES = [(1, 1), (7, 13), (33, 31), (65, 33), (64, 128), (5, 2048), (3, 2049), (2, 98432), (4096, 128)]


@pytest.mark.parametrize("form", ["per", "red", "split"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_sum_relu_add_forms(form, shape):
    rows, cols = shape
    a, b, _ = synth.sum_relu_add_inputs(rows, cols, seed=1100 + rows + cols)
    if form == "per" and cols > 2048:
        # a row the persistent form cannot hold: the forced call is refused
        with pytest.raises(fr.FrError) as e:
            gpu_sum_relu_add(a, b, form=FORMS[form])
        assert e.value.status == fr.FR_E_ARG
        return
    out = gpu_sum_relu_add(a, b, form=FORMS[form])
    _, ref = oracle.sum_relu_add(a, b)
    check_fp32(out, ref, what=f"{form} {rows}x{cols}")


@pytest.mark.parametrize("rows", [65536, 1 << 20])
def test_sum_relu_add_rows_sweep(rows):
    a, b, _ = synth.sum_relu_add_inputs(rows, 128, seed=1200)
    out = gpu_sum_relu_add(a, b)
    _, ref = oracle.sum_relu_add(a, b)
    check_fp32(out, ref, what=f"{rows}x128")


def test_sum_relu_add_strides_and_empty():
    a, b, _ = synth.sum_relu_add_inputs(10, 40, seed=1300)
    ad = dev(np.pad(a, ((0, 0), (0, 24))))[:, :40]  # row stride 64
    bd = dev(np.pad(b, ((0, 0), (0, 8))))[:, :40]  # row stride 48
    out = torch.zeros(30, dtype=torch.float32, device="cuda")
    fr.fr_sum_relu_add(ad, bd, out[::3])
    _, ref = oracle.sum_relu_add(a, b)
    got = host(out)
    check_fp32(got[::3], ref, what="strided")
    assert np.all(got[1::3] == 0) and np.all(got[2::3] == 0)
    # cols = 0: the empty sum is 0
    e = torch.empty((5, 0), dtype=torch.float32, device="cuda")
    out = torch.full((5,), 7.0, dtype=torch.float32, device="cuda")
    fr.fr_sum_relu_add(e, e, out)
    assert np.all(host(out) == 0)


# ------------------------------------------------------------------ sum of squares


@pytest.mark.parametrize("seed", [4001, 4002, 4003])
def test_sumsq_full_2_28_and_determinism(seed):
    n = 1 << 28
    x = synth.sumsq_inputs(n, seed=seed)
    xd = dev(x)
    ws = torch.empty(fr.fr_sumsq_full_workspace_bytes(n) // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    bits = set()
    for _ in range(10):
        fr.fr_sumsq_full(xd, out, ws=ws)
        bits.add(int(host(out).view(np.uint32)[0]))
    assert len(bits) == 1, "repeated runs must be bit-identical"
    ref = oracle.sumsq(x)
    got = float(host(out)[0])
    assert abs(got - ref) <= 1e-5 * ref + 1e-6, (got, ref)


_CHILD = """
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
import synth, pointwise_reduction_amd as fr
n = 1 << 28
x = torch.from_numpy(synth.sumsq_inputs(n, seed=4001)).cuda()
ws = torch.empty(fr.fr_sumsq_full_workspace_bytes(n) // 4, dtype=torch.float32, device="cuda")
out = torch.zeros(1, dtype=torch.float32, device="cuda")
fr.fr_sumsq_full(x, out, ws=ws)
print(int(out.cpu().numpy().view(np.uint32)[0]))
"""


def test_sumsq_full_bits_across_processes():
    # the same bits in separate processes (each one its own HIP context), as
    # in repeated launches of one process
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    n = 1 << 28
    xd = dev(synth.sumsq_inputs(n, seed=4001))
    ws = torch.empty(fr.fr_sumsq_full_workspace_bytes(n) // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    fr.fr_sumsq_full(xd, out, ws=ws)
    mine = int(host(out).view(np.uint32)[0])
    for _ in range(2):
        r = subprocess.run([sys.executable, "-c", _CHILD.format(root=root)], capture_output=True, text=True,
                           timeout=240)
        assert r.returncode == 0, r.stderr[-2000:]
        assert int(r.stdout.strip().splitlines()[-1]) == mine


@pytest.mark.parametrize("n", [0, 1, 7, 2048, 2049, 98432, 1 << 24, 1 << 28])
def test_sumsq_full_of_ones_is_exact(n):
    xd = torch.ones(n, dtype=torch.float32, device="cuda")
    need = fr.fr_sumsq_full_workspace_bytes(n)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda") if need else None
    out = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    fr.fr_sumsq_full(xd, out, ws=ws)
    assert float(host(out)[0]) == float(n)


def test_sumsq_closed_form_small():
    # x_i = i (n = 10): 285; x_i = i mod 8 (n = 100000, split): 140 per period.
    # Every partial sum is an integer below 2^24, so fp32 is exact.
    for x, want in ((np.arange(10, dtype=np.float32), 285.0),
                    ((np.arange(100000) % 8).astype(np.float32), 140.0 * 12500)):
        n = x.size
        out = torch.zeros(1, dtype=torch.float32, device="cuda")
        need = fr.fr_sumsq_full_workspace_bytes(n)
        ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda") if need else None
        fr.fr_sumsq_full(dev(x), out, ws=ws)
        assert float(host(out)[0]) == want


@pytest.mark.parametrize("form", ["per", "red", "split"])
def test_sumsq_rows_example_6_2(form, golden):
    g = golden("stax4_example_6_2.txt")
    rows, cols = int(g["rows"]), int(g["cols"])
    if form == "per":
        cols = 2048  # the persistent form holds at most 2048 floats per row
    x = synth.uniform((rows, cols), seed=62)
    out = torch.zeros(rows, dtype=torch.float32, device="cuda")
    with forced(FORMS[form]):
        fr.fr_sumsq_rows(dev(x), out, ws=ws_for(rows, cols))
    ref = oracle.sumsq_rows(x)
    check_fp32(host(out), ref, what=f"sumsq rows {form}")
