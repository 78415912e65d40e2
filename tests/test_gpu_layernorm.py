"""GPU parity: fr_layernorm_rows against the fp64 oracle.

bf16 in and out, fp32 arithmetic. Each output must be within one bf16 ulp of
the oracle's bf16 value (the oracle rounds its fp64 result once; the kernel
rounds an fp32 result), or - where y is a near-cancellation of its terms -
within 1e-5 * (|(x - mu) * rstd * gamma| + |beta|) + 1e-6 of the exact
value. Bit-exact pin: a constant row gives exactly beta.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_of, bf16_bits_tensor, bf16_to_f64, check_bf16, forced, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402

FORMS = {"per": fr.FR_FORM_PER, "red": fr.FR_FORM_RED}


def gpu_ln(x_bits, g_bits, b_bits, form=fr.FR_FORM_AUTO, eps=1e-5):
    x = bf16_bits_tensor(x_bits)
    y = torch.empty_like(x)
    g = None if g_bits is None else bf16_bits_tensor(g_bits)
    b = None if b_bits is None else bf16_bits_tensor(b_bits)
    with forced(form):
        fr.fr_layernorm_rows(x, y, gamma=g, beta=b, eps=eps)
    return bf16_bits_of(y)


def compare(x, g, b, got, rows=None, eps=1e-5, what=""):
    xs = x if rows is None else x[rows]
    gs = got if rows is None else got[rows]
    ref, y64, mag = oracle.layernorm_rows(xs, g, b, eps=eps)
    check_bf16(gs, ref, y64, mag, what=what)


@functools.lru_cache(maxsize=1)
def full_case(seed):
    """The 2048 x 32768 workload and its oracle result (kept for the next form)."""
    x, g, b = synth.layernorm_inputs(2048, 32768, seed=seed)
    return (x, g, b) + oracle.layernorm_rows(x, g, b)


@pytest.mark.parametrize("form", ["auto", "red"])
@pytest.mark.parametrize("seed", [3001, 3002, 3003])
def test_layernorm_2048x32768_full(form, seed):
    """Every row of the full workload, at three seeds: the automatic plan (the
    launch the benchmark times) and the looped form."""
    x, g, b, ref, y64, mag = full_case(seed)
    got = gpu_ln(x, g, b, form=fr.FR_FORM_AUTO if form == "auto" else FORMS[form])
    check_bf16(got, ref, y64, mag, what=f"2048x32768 {form} seed {seed}")


SHAPES = [(1, 8), (7, 13), (33, 31), (65, 33), (4, 4096), (3, 1000), (5, 32768), (2, 40000), (3, 16385)]


@pytest.mark.parametrize("form", ["per", "red"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_layernorm_forms(form, shape):
    rows, cols = shape
    plan_ok = cols <= (32768 if cols % 8 == 0 else 16384)
    x, g, b = synth.layernorm_inputs(rows, cols, seed=3100 + cols)
    if form == "per" and not plan_ok:
        # a row the persistent form cannot hold: the forced call is refused
        # before any launch
        with pytest.raises(fr.FrError) as e:
            gpu_ln(x, g, b, form=FORMS[form])
        assert e.value.status == fr.FR_E_ARG
        return
    got = gpu_ln(x, g, b, form=FORMS[form])
    compare(x, g, b, got, what=f"{form} {rows}x{cols}")


@pytest.mark.parametrize("form", ["per", "red"])
def test_layernorm_constant_row_is_beta(form):
    for cols in (8, 1000, 4096, 32768):
        x, g, b = synth.layernorm_inputs(2, cols, seed=3200)
        x[:] = synth.to_bf16(np.full((2, cols), -2.5625, dtype=np.float32))
        got = gpu_ln(x, g, b, form=FORMS[form])
        assert np.array_equal(got, np.broadcast_to(b, got.shape)), f"{form} cols={cols}"


@pytest.mark.parametrize("shape", [(16, 3000), (8, 4096), (4, 32768)], ids=["16x3000", "8x4096", "4x32768"])
def test_layernorm_without_affine_and_eps(shape):
    """gamma and/or beta absent (1 and 0), on masked rows and on rows that
    fill a workgroup exactly (the buffer-resource path)."""
    x, g, b = synth.layernorm_inputs(*shape, seed=3300 + shape[1])
    for eps in (1e-5, 0.0, 1.0):
        got = gpu_ln(x, None, None, eps=eps)
        compare(x, None, None, got, eps=eps, what=f"no affine eps={eps}")
    compare(x, g, None, gpu_ln(x, g, None), what="gamma only")
    compare(x, None, b, gpu_ln(x, None, b), what="beta only")


def test_layernorm_row_stride():
    x, g, b = synth.layernorm_inputs(6, 1000, seed=3400)
    xp = np.zeros((6, 1024), dtype=np.uint16)
    xp[:, :1000] = x
    xd = bf16_bits_tensor(xp)[:, :1000]
    y = torch.zeros((6, 1024), dtype=torch.bfloat16, device="cuda")
    fr.fr_layernorm_rows(xd, y[:, :1000], gamma=bf16_bits_tensor(g), beta=bf16_bits_tensor(b))
    got = bf16_bits_of(y)
    assert np.all(got[:, 1000:] == 0)
    compare(x, g, b, np.ascontiguousarray(got[:, :1000]), what="row stride 1024")


@pytest.mark.parametrize("nr", [3, 5, 8])
def test_layernorm_pipelined_rows(nr):
    """The pipelined form (a workgroup takes nr rows, 3 in flight, gamma and
    beta staged in LDS) through a tuner override, on 300 rows: at nr = 8 the
    last workgroup has 4 rows past the end, which touch no memory. Every row
    against the oracle, with and without gamma / beta, in place, and the same
    bits (outputs and row statistics) as one row per workgroup, which is the
    automatic plan below 3 rows per CU."""
    rows, cols = 300, 32768
    x, g, b = synth.layernorm_inputs(rows, cols, seed=3500 + nr)
    xd, gd, bd = bf16_bits_tensor(x), bf16_bits_tensor(g), bf16_bits_tensor(b)
    assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, rows, cols, dtype=fr.FR_BF16).rows_per_wg == 1

    def run(gamma, beta, pipelined, in_place=False):
        y = xd.clone() if in_place else torch.full_like(xd, float("nan"))
        mean = torch.full((rows,), float("nan"), device="cuda")
        rstd = torch.full((rows,), float("nan"), device="cuda")
        if pipelined:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=512, vec=8, rows_per_wg=nr)
        try:
            assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, rows, cols, dtype=fr.FR_BF16).rows_per_wg == \
                (nr if pipelined else 1)
            fr.fr_layernorm_rows_stats(y if in_place else xd, y, mean=mean, rstd=rstd, gamma=gamma, beta=beta)
        finally:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM)
        return bf16_bits_of(y), host(mean), host(rstd)

    for gamma, beta, what in ((gd, bd, "affine"), (None, None, "no affine"), (gd, None, "gamma only"),
                              (None, bd, "beta only")):
        got, mean, rstd = run(gamma, beta, True)
        gh = None if gamma is None else g
        bh = None if beta is None else b
        compare(x, gh, bh, got, what=f"pipelined nr={nr} {what}")
        ref, ref_mean, ref_rstd = run(gamma, beta, False)
        assert np.array_equal(got, ref), f"pipelined nr={nr} {what}: bits differ from one row per workgroup"
        assert np.array_equal(mean.view(np.uint32), ref_mean.view(np.uint32))
        assert np.array_equal(rstd.view(np.uint32), ref_rstd.view(np.uint32))
    m64, r64 = oracle.layernorm_stats(x)
    assert np.allclose(mean, m64, rtol=1e-5, atol=1e-6) and np.allclose(rstd, r64, rtol=1e-5)
    got, _, _ = run(gd, bd, True, in_place=True)
    compare(x, g, b, got, what=f"pipelined nr={nr} in place")


@pytest.mark.parametrize("form", ["per", "pipelined", "red"])
@pytest.mark.parametrize("cols", [1000, 32768])
def test_layernorm_nan_and_inf_rows(form, cols):
    """A NaN or an infinity anywhere in a row makes every output of that row
    NaN (the mean is NaN or infinite, and x - mean is NaN); the other rows
    are untouched. Through each form, including the dot-product row sum."""
    x, g, b = synth.layernorm_inputs(4, cols, seed=3600 + cols)
    if form == "pipelined" and cols != 32768:
        # the pipelined form takes rows of 32768 only: a candidate plan that
        # asks for it on other rows is refused
        fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=512, vec=8, rows_per_wg=3)
        try:
            with pytest.raises(fr.FrError) as e:
                gpu_ln(x, g, b)
        finally:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM)
        assert e.value.status == fr.FR_E_ARG
        return
    special = {0: 0x7FC0, 1: 0x7F80, 2: 0xFF80}  # NaN, +inf, -inf at a different column each
    for r, bits in special.items():
        x[r, (r * 977 + 5) % cols] = bits
    if form == "pipelined":
        fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=512, vec=8, rows_per_wg=3)
        try:
            got = gpu_ln(x, g, b)
        finally:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM)
    else:
        got = gpu_ln(x, g, b, form=FORMS[form])
    vals = bf16_to_f64(got)
    assert np.isnan(vals[:3]).all(), f"{form} {cols}: rows with NaN or inf must be all NaN"
    compare(x[3:], g, b, got[3:], what=f"{form} {cols} clean row")


@pytest.mark.parametrize("rows", [1001, 4096])
def test_layernorm_pipelined_automatic_row_counts(rows):
    """The automatic plan at row counts other than the workload's: 1001 rows
    (4 per workgroup, 251 workgroups, the last one with a row past the end)
    and 4096 rows (8 per workgroup, 512 workgroups: two rounds of one
    workgroup per CU). 1001: every row against the oracle; 4096: every 7th
    row and the last."""
    cols = 32768
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, rows, cols, dtype=fr.FR_BF16,
                         num_cus=torch.cuda.get_device_properties(0).multi_processor_count)
    assert p.rows_per_wg > 1
    x, g, b = synth.layernorm_inputs(rows, cols, seed=3700 + rows)
    got = gpu_ln(x, g, b)
    pick = None if rows == 1001 else np.r_[np.arange(0, rows, 7), rows - 1]
    compare(x, g, b, got, rows=pick, what=f"pipelined {rows}x{cols}")
