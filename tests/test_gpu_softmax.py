"""GPU parity: fr_softmax_rows against the fp64 oracle.

Covers the persistent, looped and split forms (forced), the 4096 x 1024
workload in full, the ragged 512-row workload in full (lengths from
{1000, 3000, 50257, 131071}, padded to 131072, tails never read or written),
the pages' boundary shapes, bit-exact pins (argmax, constant rows) and
determinism. Tolerance per element: |y - y_ref| <= 1e-5 * y_ref + 1e-6.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_fp32, dev, forced, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402

FORMS = {"per": fr.FR_FORM_PER, "red": fr.FR_FORM_RED, "split": fr.FR_FORM_SPLIT}


def run(x_np, lengths=None, form=fr.FR_FORM_AUTO, use_ws=None, cols=None, y_fill=np.nan, argmax=True, ws_bytes=None):
    """Run the GPU softmax on x_np[:, :cols]; returns (y, argmax)."""
    rows = x_np.shape[0]
    cols = x_np.shape[1] if cols is None else cols
    xd = dev(x_np)
    x = xd[:, :cols]
    yd = torch.full(xd.shape, float(y_fill), dtype=torch.float32, device="cuda")
    y = yd[:, :cols]
    L = None if lengths is None else dev(np.asarray(lengths, dtype=np.int32))
    am = torch.full((rows,), -7, dtype=torch.int32, device="cuda") if argmax else None
    if use_ws is None:
        use_ws = form == fr.FR_FORM_SPLIT
    ws = None
    if use_ws:
        ws = new_ws(rows, cols, nbytes=ws_bytes)
    with forced(form):
        fr.fr_softmax_rows(x, y, lengths=L, argmax=am, ws=ws)
    return host(yd)[:, :cols], (host(am) if argmax else None), host(yd)


def new_ws(rows, cols, garbage=0x5A5A5A5A, init=True, nbytes=None):
    """A split workspace holding garbage, then initialized (unless init=False)."""
    nbytes = fr.fr_softmax_rows_workspace_bytes(rows, cols) if nbytes is None else nbytes
    ws = torch.full((nbytes // 4,), garbage, dtype=torch.int32, device="cuda")
    return fr.fr_softmax_rows_workspace_init(ws) if init else ws


def recomputed(ws):
    """The workspace's count of partials the single pass computed a second time."""
    return int(host(ws[:1]).view(np.uint32)[0])


def valid_mask(rows, cols, lengths):
    L = np.full(rows, cols) if lengths is None else np.clip(np.asarray(lengths, dtype=np.int64), 0, cols)
    return np.arange(cols)[None, :] < L[:, None]


def compare(x_np, y, am, lengths=None, cols=None, what=""):
    cols = x_np.shape[1] if cols is None else cols
    y64, am_ref = oracle.softmax_rows(x_np[:, :cols] if cols != x_np.shape[1] else x_np, lengths=lengths)
    written = valid_mask(x_np.shape[0], cols, lengths)  # j < len_i
    check_fp32(np.where(written, y, 0.0), np.where(written, y64, 0.0), what=what)
    if am is not None:
        assert np.array_equal(am, am_ref), f"{what}: argmax differs at rows {np.nonzero(am != am_ref)[0][:8]}"


# ------------------------------------------------------------------ the headline workload


@pytest.mark.parametrize("seed", [2001, 2002, 2003])
def test_softmax_4096x1024(seed):
    x = synth.softmax_inputs(4096, 1024, seed=seed)
    y, am, _ = run(x)
    compare(x, y, am, what=f"4096x1024 seed {seed}")
    assert np.allclose(y.sum(axis=1), 1.0, atol=1e-5)


# ------------------------------------------------------------------ forms on the pages' shapes

SMALL = [(1, 1), (7, 13), (33, 31), (65, 33), (256, 1000), (1823, 781), (3, 1024), (5, 2048), (2, 257)]


@pytest.mark.parametrize("form", ["per", "red", "split"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"{r}x{c}" for r, c in SMALL])
def test_softmax_forms_small(form, shape):
    rows, cols = shape
    x = synth.softmax_inputs(rows, cols, seed=2100 + rows + cols)
    y, am, _ = run(x, form=FORMS[form])
    compare(x, y, am, what=f"{form} {rows}x{cols}")


LONG = [2049, 4097, 8192, 8193, 20000, 50257, 131071]


@pytest.mark.parametrize("form", ["red", "split"])
@pytest.mark.parametrize("cols", LONG)
def test_softmax_forms_long_rows(form, cols):
    x = synth.softmax_inputs(3, cols, seed=2200 + cols)
    y, am, _ = run(x, form=FORMS[form])
    compare(x, y, am, what=f"{form} 3x{cols}")


@pytest.mark.parametrize("form", ["per", "red", "split"])
def test_softmax_constant_rows_are_exactly_one_over_n(form):
    lengths = [1, 3, 64, 1000, 1024, 2048] + ([5000, 50257] if form != "per" else [])
    for n in lengths:
        x = np.full((2, n), 0.3125, dtype=np.float32)
        y, am, _ = run(x, form=FORMS[form])
        assert np.all(y == np.float32(1.0) / np.float32(n)), f"{form} n={n}"
        assert np.all(am == 0)


def test_softmax_worked_example(golden):
    g = golden("hello_gpu_ch12_worked_example.txt")
    x = np.array([g["scores"]], dtype=np.float32)
    for form in ("per", "red", "split"):
        y, am, _ = run(x, form=FORMS[form])
        np.testing.assert_allclose(y[0], g["probabilities"], atol=g["tolerance"])
        assert am[0] == 2


# ------------------------------------------------------------------ ragged rows


@pytest.mark.parametrize("form", ["per", "red", "split"])
def test_softmax_ragged_small(form):
    cap = 2048 if form == "per" else 4100
    lens = [0, 1, 2, 3, 63, 64, 65, 127, 1000, 1023, 1024, 1025, 2047, 2048]
    if form != "per":
        lens += [2049, 4095, 4097, 4100]
    L = np.array(lens, dtype=np.int32)
    x, _ = synth.ragged_softmax_inputs(len(L), cap, seed=2300, lengths=L)
    y, am, yfull = run(x, lengths=L, form=FORMS[form])
    compare(x, y, am, lengths=L, what=f"ragged {form}")
    for r, n in enumerate(L):
        assert np.isnan(yfull[r, n:]).all(), f"row {r}: output tail beyond len {n} was written"
    assert am[0] == -1


def test_softmax_lengths_are_clamped():
    L = np.array([-5, 0, 40, 1 << 30], dtype=np.int32)
    x = synth.softmax_inputs(4, 40, seed=2400)
    y, am, _ = run(x, lengths=L)
    compare(x, y, am, lengths=L, what="clamped lengths")
    assert am[0] == -1 and am[1] == -1


@functools.lru_cache(maxsize=1)
def ragged_case(seed):
    """The ragged 512-row workload and its oracle result (kept for the next form)."""
    x, L = synth.ragged_softmax_inputs(512, 131072, seed=seed)
    y64, am_ref = oracle.softmax_rows(x, lengths=L)
    return x, L, y64, am_ref


@pytest.mark.parametrize("use_ws", [True, False], ids=["split", "looped"])
@pytest.mark.parametrize("seed", [5001, 5002, 5003])
def test_softmax_ragged_512x131072_full(seed, use_ws):
    """The ragged workload at full size, three seeds, in the launch the
    benchmark times (split, with a workspace) and the looped form. Input tails
    hold NaN (a read would poison the row) and the output tails hold a
    sentinel that must survive."""
    x, L, y64, am_ref = ragged_case(seed)
    sentinel = -12345.0
    y, am, yfull = run(x, lengths=L, use_ws=use_ws, y_fill=sentinel)
    plan = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, has_lengths=True,
                            ws_bytes=fr.fr_softmax_rows_workspace_bytes(512, 131072) if use_ws else 0)
    assert plan.form == (fr.FR_FORM_SPLIT if use_ws else fr.FR_FORM_RED)
    assert np.array_equal(am, am_ref)
    written = valid_mask(512, 131072, L)
    assert np.all(yfull[~written] == sentinel), "an output tail was written"
    check_fp32(np.where(written, y, 0.0), np.where(written, y64, 0.0), what=f"ragged 512x131072 seed {seed}")
    assert np.isfinite(y[written]).all()


# ------------------------------------------------------------------ semantics


def test_softmax_nan_row_and_first_argmax():
    x = synth.softmax_inputs(6, 300, seed=2500)
    x[1, 17] = np.nan
    x[2, 5] = x[2].max() + 1
    x[2, 250] = x[2, 5]  # tie: the first index wins
    x[3, :] = -np.inf
    x[4, 10] = np.inf
    for form in ("per", "red", "split"):
        y, am, _ = run(x, form=FORMS[form])
        compare(x, y, am, what=f"special values {form}")
        assert am[1] == 17 and am[2] == 5 and np.isnan(y[1]).all()


def test_softmax_in_place_and_row_stride():
    x = synth.softmax_inputs(64, 1000, seed=2600)
    xd = dev(np.pad(x, ((0, 0), (0, 24))))  # row stride 1024, 24 padding columns
    view = xd[:, :1000]
    fr.fr_softmax_rows(view, view)  # in place
    y = host(xd)
    assert np.all(y[:, 1000:] == 0)
    y64, _ = oracle.softmax_rows(x)
    check_fp32(y[:, :1000], y64, what="in place, strided")


def test_softmax_unaligned_rows_use_element_path():
    x = synth.softmax_inputs(9, 1001, seed=2700)
    xd = dev(x)  # row stride 1001: rows are not 16-byte aligned
    y = torch.empty_like(xd)
    am = torch.empty(9, dtype=torch.int32, device="cuda")
    for form in ("per", "red"):
        with forced(FORMS[form]):
            fr.fr_softmax_rows(xd, y, argmax=am)
        compare(x, host(y), host(am), what=f"unaligned {form}")


@pytest.mark.parametrize("passes", [1, 2])
def test_softmax_unaligned_rows_split(passes):
    """Rows that are not 16-byte aligned (row stride 20001 floats) through
    both split variants: the element-wise path of each kernel (the single pass
    then keeps one chunk in registers and reads it with masked loads)."""
    x, L = synth.ragged_softmax_inputs(7, 20001, seed=2710, choices=(1, 8193, 19999, 20001))
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=passes)
        y, am, yfull = run(x, lengths=L, use_ws=True)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    compare(x, y, am, lengths=L, what=f"unaligned split passes={passes}")
    for r, n in enumerate(L):
        assert np.isnan(yfull[r, n:]).all()


@pytest.mark.parametrize("seed", [3101, 3102, 3103])
def test_softmax_single_pass_random_ragged(seed):
    """Seeded random shapes through the single pass: row counts, capacities
    and lengths drawn around the chunk size (8192), with empty rows, rows of
    one element and rows that end one element before or after a chunk edge."""
    rng = np.random.default_rng(seed)
    rows = int(rng.integers(1, 200))
    cols = int(rng.integers(8193, 160000))
    edges = [0, 1, 8191, 8192, 8193, 16383, 16385, cols - 1, cols]
    L = np.where(rng.random(rows) < 0.5, rng.choice(edges, rows), rng.integers(0, cols + 1, rows))
    L = np.clip(L, 0, cols).astype(np.int32)
    x, _ = synth.ragged_softmax_inputs(rows, cols, seed=seed, lengths=L)
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=1)
        y, am, yfull = run(x, lengths=L, use_ws=True)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    compare(x, y, am, lengths=L, what=f"single pass {rows}x{cols} seed {seed}")
    for r, n in enumerate(L):
        assert np.isnan(yfull[r, n:]).all(), f"row {r}: output tail beyond len {n} was written"


def test_softmax_single_pass_most_rows():
    """The largest row count the single pass takes (its chunk list lives in
    LDS): 2048 rows, each thread of the list scan counting 8 of them."""
    rows, cols = 2048, 9000
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=3110, choices=(0, 1, 4000, 8192, 8193, 9000))
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=1)
        y, am, _ = run(x, lengths=L, use_ws=True)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    compare(x, y, am, lengths=L, what="single pass 2048 rows")


def test_softmax_single_pass_graph_replays():
    # the slot reset is a fill kernel, so the single pass can be recorded in
    # a graph: every replay (after an eager call on other data through the
    # same workspace, and a synchronisation) equals the eager result bit for bit
    rows, cols = 96, 131072
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=2860)
    x2, L2 = synth.ragged_softmax_inputs(rows, cols, seed=2861)
    xd, Ld, x2d, L2d = dev(x), dev(L), dev(x2), dev(L2)
    ws = new_ws(rows, cols)
    y, y2 = torch.full_like(xd, float("nan")), torch.empty_like(xd)
    am = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    am2 = torch.empty_like(am)

    def call():
        fr.fr_softmax_rows(xd, y, lengths=Ld, argmax=am, ws=ws)

    call()
    torch.cuda.synchronize()
    ref_y, ref_am = host(y), host(am)
    compare(x, ref_y, ref_am, lengths=L, what="eager single pass")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    valid = valid_mask(rows, cols, L)
    for rep in range(4):
        y.fill_(0.0)
        am.fill_(-7)
        fr.fr_softmax_rows(x2d, y2, lengths=L2d, argmax=am2, ws=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        yr = host(y)
        assert np.array_equal(yr[valid].view(np.uint32), ref_y[valid].view(np.uint32)), rep
        assert np.array_equal(host(am), ref_am), rep


def test_softmax_is_deterministic():
    x, L = synth.ragged_softmax_inputs(64, 60000, seed=2800, choices=(1000, 59999, 60000))
    outs = [run(x, lengths=L, use_ws=True)[2] for _ in range(3)]
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


@pytest.mark.parametrize("passes", [1, 2])
@pytest.mark.parametrize("cols", [8193, 50257, 131071, 140000, 600001])
def test_softmax_split_passes(passes, cols):
    """Both split variants: one read with the row's partials exchanged inside
    one kernel, and the partial + finishing kernels. 600001 columns make 74
    chunks per row (more than one 64-lane merge group)."""
    rows = 24 if cols < 600000 else 5
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=2900 + cols, choices=(1, 4000, cols - 7, cols))
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=passes)
        y, am, yfull = run(x, lengths=L, use_ws=True)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    compare(x, y, am, lengths=L, what=f"split passes={passes} cols={cols}")
    for r, n in enumerate(L):
        assert np.isnan(yfull[r, n:]).all()


@pytest.mark.parametrize("vec,cols", [(4, 40000), (8, 20000)])
def test_softmax_single_pass_many_rounds(vec, cols):
    """2048 ragged rows: the chunk list runs over many rounds of the grid
    (entries w, w + G, ... per workgroup); at 40000 columns in chunks of 4096
    a workgroup takes about 10 entries, past the ones whose rows are found
    while the list is built. The single pass matches the oracle and the
    two-kernel form's argmax, and empty rows get -1."""
    rows = 2048
    rng = np.random.default_rng(2950 + vec)
    L = rng.integers(0, cols + 1, size=rows).astype(np.int32)
    L[rng.random(rows) < 0.05] = 0
    x = synth.normal((rows, cols), seed=2950 + vec) * 3
    outs = {}
    try:
        for passes in (1, 2):
            fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=vec, passes=passes)
            need = fr.fr_plan_query(fr.FR_OP_SOFTMAX, rows, cols, has_lengths=True, ws_bytes=1 << 40).ws_bytes
            outs[passes] = run(x, lengths=L, use_ws=True, ws_bytes=need)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    y, am, yfull = outs[1]
    compare(x, y, am, lengths=L, what=f"single pass, vec {vec}")
    assert np.array_equal(am, outs[2][1])
    assert np.all(am[L == 0] == -1)
    for r in np.nonzero(L < cols)[0][:64]:
        assert np.isnan(yfull[r, L[r]:]).all()


@pytest.mark.parametrize("shape", [(64, 131072), (3, 600001), (7, 20001)], ids=["64x131072", "3x600001", "7x20001"])
def test_softmax_single_pass_fallback_gives_the_same_bits(shape):
    """In the single pass a workgroup that stops waiting computes the missing
    partials of its row from x itself. Forced for every partial (wait_us < 0),
    y and the argmax keep their bits, and the workspace's count grows by each
    recomputed partial: sum over rows of nc * (nc - 1). 7 x 20001 has rows
    that are not 16-byte aligned (row stride 20001 floats): the element-wise
    path, whose recompute streams the chunk instead of taking it from
    registers. The workspace held garbage before its initialization. How
    many partials the default wait recomputed depends on scheduling (a busy
    device makes partners late), so it is reported, not asserted."""
    rows, cols = shape
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=2950 + rows, choices=(1000, cols // 2 + 3, cols - 1, cols))
    xd, Ld = dev(x), dev(L)
    ws = new_ws(rows, cols)
    outs = {}
    try:
        for wait in (0, -1):
            fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=1, wait_us=wait)
            y = torch.full_like(xd, float("nan"))
            am = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
            before = recomputed(ws)
            fr.fr_softmax_rows(xd, y, lengths=Ld, argmax=am, ws=ws)
            outs[wait] = (host(y), host(am), recomputed(ws) - before)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    nc = (np.asarray(L, dtype=np.int64) + 8191) // 8192
    print(f"{rows}x{cols}: {outs[0][2]} partials recomputed with the default wait")
    assert outs[-1][2] == int((nc * (nc - 1)).sum())
    assert np.array_equal(outs[0][0].view(np.uint32), outs[-1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[-1][1])
    compare(x, outs[0][0], outs[0][1], lengths=L, what=f"single pass {rows}x{cols}")


def one_call(x, L, ws, passes=1, vec=8, argmax=True):
    xd, Ld = dev(x), dev(L)
    y = torch.full_like(xd, float("nan"))
    am = torch.full((x.shape[0],), -7, dtype=torch.int32, device="cuda") if argmax else None
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=vec, passes=passes)
        fr.fr_softmax_rows(xd, y, lengths=Ld, argmax=am, ws=ws)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    return host(y), (host(am) if argmax else None)


def test_softmax_single_pass_workspace_reused_across_calls():
    """One workspace, initialized once, through a sequence of calls whose
    chunk lists differ (row counts, lengths, chunk sizes, the two-kernel form
    in between): slots left by an earlier call carry that call's tag (or the
    two-kernel form's), which the next call never accepts. Every call equals,
    bit for bit, the same call on a freshly initialized workspace, and the
    oracle."""
    cap = 131072
    big = fr.fr_softmax_rows_workspace_bytes(96, cap)
    for vec in (4,):
        big = max(big, 64 + 96 * (cap // (256 * 4 * vec)) * 16)
    ws = fr.fr_softmax_rows_workspace_init(torch.full((big // 4,), 0x7F7F7F7F, dtype=torch.int32, device="cuda"))
    calls = [(96, (131071, 50257, 3000), 1, 8), (40, (131072, 9000), 1, 8), (96, (131071, 70000, 1000), 2, 8),
             (96, (131071, 50257, 3000), 1, 8), (17, (100000, 30000, 8193), 1, 4), (96, (120000, 1), 1, 8),
             (40, (131072, 9000), 1, 8)]
    for i, (rows, choices, passes, vec) in enumerate(calls):
        x, L = synth.ragged_softmax_inputs(rows, cap, seed=3200 + i, choices=choices)
        y, am = one_call(x, L, ws, passes=passes, vec=vec)
        fresh = fr.fr_softmax_rows_workspace_init(torch.empty(big // 4, dtype=torch.int32, device="cuda"))
        y0, am0 = one_call(x, L, fresh, passes=passes, vec=vec)
        written = valid_mask(rows, cap, L)
        assert np.array_equal(y[written].view(np.uint32), y0[written].view(np.uint32)), f"call {i}"
        assert np.array_equal(am, am0), f"call {i}"
        compare(x, y, am, lengths=L, what=f"reused workspace, call {i}")
        assert np.isnan(y[~written]).all(), f"call {i}: an output tail was written"


def test_softmax_single_pass_uninitialized_workspace_is_still_exact():
    """A workspace that was never initialized (no mark in its header) is
    never trusted: every partner partial is computed from x, giving the same
    bits as an initialized workspace, and the count grows by sum nc * (nc - 1)."""
    rows, cols = 48, 131072
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=3300)
    good = new_ws(rows, cols)
    y0, am0 = one_call(x, L, good)
    for garbage in (0x5A5A5A5A, 0, -1):
        bad = new_ws(rows, cols, garbage=garbage, init=False)
        before = recomputed(bad)
        y, am = one_call(x, L, bad)
        nc = (np.asarray(L, dtype=np.int64) + 8191) // 8192
        assert (recomputed(bad) - before) % (1 << 32) == int((nc * (nc - 1)).sum()), hex(garbage & 0xFFFFFFFF)
        written = valid_mask(rows, cols, L)
        assert np.array_equal(y[written].view(np.uint32), y0[written].view(np.uint32))
        assert np.array_equal(am, am0)


def test_softmax_single_pass_epoch_limit():
    """The call counter is 31 bits: the call that takes the last tag still
    exchanges partials; from the next call on no slot is trusted (same bits,
    every partner partial recomputed) until the workspace is initialized
    again. The counter is set near its end through the header word that
    holds it (word 2)."""
    rows, cols = 32, 131072
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=3400)
    nc = (np.asarray(L, dtype=np.int64) + 8191) // 8192
    ws = new_ws(rows, cols)
    y0, am0 = one_call(x, L, ws)
    ws[2] = 0x7FFFFFFE  # the last call that may take a tag
    written = valid_mask(rows, cols, L)
    for expect_all in (False, True):
        before = recomputed(ws)
        y, am = one_call(x, L, ws)
        delta = recomputed(ws) - before
        if expect_all:
            assert delta == int((nc * (nc - 1)).sum())
        assert np.array_equal(y[written].view(np.uint32), y0[written].view(np.uint32))
        assert np.array_equal(am, am0)
    assert int(host(ws[2:3])[0]) == 0x7FFFFFFF
    fr.fr_softmax_rows_workspace_init(ws)
    assert int(host(ws[2:3])[0]) == 0
    y, am = one_call(x, L, ws)
    assert np.array_equal(y[written].view(np.uint32), y0[written].view(np.uint32))
    assert int(host(ws[2:3])[0]) == 1


@pytest.mark.parametrize("wait", [0, -1])
def test_softmax_split_in_place(wait):
    """y == x through the split form. The single pass could recompute a late
    partner's partial from a chunk that partner has already overwritten, so
    an in-place call takes the two-kernel split and matches the oracle; a
    tuning override that forces the single pass in place is refused."""
    rows, cols = 24, 50000
    x, L = synth.ragged_softmax_inputs(rows, cols, seed=2970, choices=(1000, 8193, 40000, 50000))
    Ld = dev(L)
    ws = new_ws(rows, cols)
    am = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    xd = dev(x)
    with forced(fr.FR_FORM_SPLIT):
        fr.fr_softmax_rows(xd, xd, lengths=Ld, argmax=am, ws=ws)
    y = host(xd)
    compare(x, y, host(am), lengths=L, what="split in place (automatic)")
    written = valid_mask(rows, cols, L)
    assert np.isnan(y[~written]).all(), "an input tail was written"
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=2, wait_us=wait)
        xd = dev(x)
        fr.fr_softmax_rows(xd, xd, lengths=Ld, argmax=am, ws=ws)
        compare(x, host(xd), host(am), lengths=L, what="split in place (two kernels)")
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=1, wait_us=wait)
        xd = dev(x)
        with pytest.raises(fr.FrError):
            fr.fr_softmax_rows(xd, xd, lengths=Ld, argmax=am, ws=ws)
        assert np.array_equal(host(xd).view(np.uint32), x.view(np.uint32)), "a refused call wrote y"
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
