"""GPU parity: LayerNorm statistics and backward against the fp64 oracle.

fr_layernorm_rows_stats writes the mean and rstd each row used: within
1e-5 * (mean of |x|) + 1e-6 (mean) and 1e-5 relative (rstd) of the oracle's
fp64 statistics, and y bit-identical to fr_layernorm_rows.

fr_layernorm_rows_backward reads saved statistics. Both sides get the same
fp32 mean and rstd (the oracle's statistics rounded to fp32, never the
library's). dx (bf16): within one bf16 ulp of the oracle's rounded value, or
within 1e-5 * rstd (|g_j| + mean|g| + |xh_j| mean|g xh|) + 1e-6 of the exact
value where dx is a near-cancellation. dgamma, dbeta (fp32): within 1e-5 *
sum_i |terms| + 1e-6. Inputs: x, gamma as for the LayerNorm forward
(x ~ N(0.5, 2^2), gamma ~ U(0.5, 1.5), bf16), dy ~ N(0, 1) bf16.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_of, bf16_bits_tensor, check_bf16, check_fp32, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


def inputs(rows, cols, seed):
    x, g, _ = synth.layernorm_inputs(rows, cols, seed=seed)
    dy = synth.to_bf16(synth.normal((rows, cols), seed, stream=5))
    mean, rstd = oracle.layernorm_stats(x, eps=1e-5)
    return x, dy, g, mean.astype(np.float32), rstd.astype(np.float32)


def run_bwd(x, dy, g, mean, rstd, want_dg=True, offset=0, inplace=False, ws=None):
    """Device call; offset > 0 shifts x, dy, dx by that many elements (element accesses)."""
    rows, cols = x.shape

    def place(bits):
        if offset == 0:
            return bf16_bits_tensor(bits)
        flat = np.concatenate([np.zeros(offset, np.uint16), bits.ravel()])
        return bf16_bits_tensor(flat)[offset:].view(rows, cols)
    xd, dyd = place(x), place(dy)
    dxd = dyd if inplace else place(np.full_like(x, 0x7FC0))
    gd = None if g is None else bf16_bits_tensor(g)
    dg = torch.full((cols,), np.nan, dtype=torch.float32, device="cuda") if want_dg else None
    db = torch.full((cols,), np.nan, dtype=torch.float32, device="cuda") if want_dg else None
    fr.fr_layernorm_rows_backward(xd, dyd, dev(mean), dev(rstd), dxd, gamma=gd, dgamma=dg, dbeta=db, ws=ws)
    out = {"dx": bf16_bits_of(dxd)}
    if want_dg:
        out["dgamma"], out["dbeta"] = host(dg), host(db)
    return out


def compare(x, dy, g, mean, rstd, got, what=""):
    ref = oracle.layernorm_backward_rows(x, dy, g, mean.astype(np.float64), rstd.astype(np.float64))
    check_bf16(got["dx"], oracle.round_bf16(ref["dx64"]), ref["dx64"], ref["dxmag"], what=what + " dx")
    if "dgamma" in got:
        check_fp32(got["dgamma"], ref["dgamma64"], terms=ref["gmag"], what=what + " dgamma")
        check_fp32(got["dbeta"], ref["dbeta64"], terms=ref["bmag"], what=what + " dbeta")


# shapes across every compiled geometry: 128 x 1 up to 1024 x 4 vectors of 8,
# whole rows, rows with a masked last vector, and many rows per workgroup
SHAPES = [(1, 8), (3, 1000), (5, 1024), (7, 3000), (16, 4096), (8, 8192), (3, 16384), (2, 20000), (2, 32768),
          (300, 1000), (5000, 256), (600, 32768)]


@pytest.mark.parametrize("shape", SHAPES)
def test_layernorm_backward_shapes(shape):
    x, dy, g, mean, rstd = inputs(*shape, seed=shape[0] * 31 + shape[1])
    compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd), what=str(shape))


@pytest.mark.parametrize("shape", [(4, 1000), (9, 4096), (3, 24576)])
def test_layernorm_backward_without_gamma_or_column_sums(shape):
    x, dy, g, mean, rstd = inputs(*shape, seed=7)
    compare(x, dy, None, mean, rstd, run_bwd(x, dy, None, mean, rstd), what="no gamma")
    compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, want_dg=False), what="dx only")


@pytest.mark.parametrize("shape", [(5, 1003), (4, 4096), (3, 16000), (2, 30001)])
def test_layernorm_backward_element_accesses(shape):
    # odd lengths and unaligned bases: element loads and stores; beyond 16384
    # columns the column sums need 16-byte accesses
    x, dy, g, mean, rstd = inputs(*shape, seed=11)
    if shape[1] > 16384:
        with pytest.raises(fr.FrError) as ei:
            run_bwd(x, dy, g, mean, rstd, offset=1)
        assert ei.value.status == fr.FR_E_ALIGN
        compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, offset=1, want_dg=False), what="unaligned dx")
    else:
        compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, offset=1), what=f"unaligned {shape}")


def test_layernorm_backward_in_place_and_deterministic():
    x, dy, g, mean, rstd = inputs(64, 4096, seed=13)
    a = run_bwd(x, dy, g, mean, rstd)
    b = run_bwd(x, dy, g, mean, rstd, inplace=True)
    assert np.array_equal(a["dx"], b["dx"])
    assert np.array_equal(a["dgamma"], b["dgamma"]) and np.array_equal(a["dbeta"], b["dbeta"])
    compare(x, dy, g, mean, rstd, a, what="64x4096")


def test_layernorm_backward_errors_and_empty():
    x, dy, g, mean, rstd = inputs(4, 1024, seed=17)
    with pytest.raises(fr.FrError) as ei:
        run_bwd(x, dy, g, mean, rstd, ws=torch.empty(4, dtype=torch.float32, device="cuda"))
    assert ei.value.status == fr.FR_E_WORKSPACE
    big = torch.zeros((2, 32776), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(2, dtype=torch.float32, device="cuda")
    with pytest.raises(fr.FrError) as ei:
        fr.fr_layernorm_rows_backward(big, big, st, st, big)
    assert ei.value.status == fr.FR_E_SIZE
    # no rows: dgamma and dbeta are empty sums
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dg = torch.full((64,), 5.0, dtype=torch.float32, device="cuda")
    db = torch.full((64,), 5.0, dtype=torch.float32, device="cuda")
    fr.fr_layernorm_rows_backward(e, e, st[:0], st[:0], e, dgamma=dg, dbeta=db)
    assert np.all(host(dg) == 0.0) and np.all(host(db) == 0.0)


@pytest.mark.parametrize("shape", [(16, 3000), (8, 4096), (4, 32768), (3, 50000)])
def test_layernorm_stats_output(shape):
    rows, cols = shape
    x, g, b = synth.layernorm_inputs(rows, cols, seed=19)
    xd = bf16_bits_tensor(x)
    y1, y2 = torch.empty_like(xd), torch.empty_like(xd)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    gd, bd = bf16_bits_tensor(g), bf16_bits_tensor(b)
    fr.fr_layernorm_rows(xd, y1, gamma=gd, beta=bd)
    fr.fr_layernorm_rows_stats(xd, y2, mean=mean, rstd=rstd, gamma=gd, beta=bd)
    assert np.array_equal(bf16_bits_of(y1), bf16_bits_of(y2))
    m64, r64 = oracle.layernorm_stats(x, eps=1e-5)
    xa = np.abs((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)).mean(axis=1)
    assert np.all(np.abs(host(mean) - m64) <= 1e-5 * xa + 1e-6)
    assert np.all(np.abs(host(rstd) - r64) <= 1e-5 * r64)


def test_layernorm_backward_full_size():
    # 2048 x 32768 bf16 with gamma: the benchmark's launch (split rows, a
    # team of 4 workgroups per row). Every output against the oracle.
    rows, cols = 2048, 32768
    x, dy, g, mean, rstd = inputs(rows, cols, seed=3001)
    got = run_bwd(x, dy, g, mean, rstd)
    ref = oracle.layernorm_backward_rows(x, dy, g, mean.astype(np.float64), rstd.astype(np.float64))
    check_fp32(got["dgamma"], ref["dgamma64"], terms=ref["gmag"], what="full dgamma")
    check_fp32(got["dbeta"], ref["dbeta64"], terms=ref["bmag"], what="full dbeta")
    check_bf16(got["dx"], oracle.round_bf16(ref["dx64"]), ref["dx64"], ref["dxmag"], what="full dx")
    # the persistent form on the same inputs (dx overwrites dy: no split)
    got2 = run_bwd(x, dy, g, mean, rstd, inplace=True)
    check_bf16(got2["dx"], oracle.round_bf16(ref["dx64"]), ref["dx64"], ref["dxmag"], what="full dx, persistent")
    check_fp32(got2["dgamma"], ref["dgamma64"], terms=ref["gmag"], what="full dgamma, persistent")


# ---- split rows: a team of workgroups per row (rows longer than 8192 columns)

def team_ws(rows, cols, init=True):
    n = fr.fr_layernorm_rows_backward_workspace_bytes(rows, cols)
    ws = torch.zeros(n // 4, dtype=torch.float32, device="cuda")
    if init:
        fr.fr_layernorm_rows_backward_workspace_init(ws)
    return ws


def recomputed(ws):
    """The workspace's cumulative count of partner sums a member computed
    itself (header word 0)."""
    return int(ws[:1].view(torch.int32).item()) & 0xFFFFFFFF


@pytest.mark.parametrize("shape", [(1, 8200), (3, 16384), (7, 20000), (5, 24576), (9, 32768), (300, 16392),
                                   (257, 32768)])
def test_layernorm_backward_split_rows(shape):
    # forced split form: 2, 3 and 4 parts, a narrower last part, fewer rows
    # than teams and more, with and without gamma and the column sums
    x, dy, g, mean, rstd = inputs(*shape, seed=shape[0] * 7 + shape[1])
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        p = fr.fr_plan_query(fr.FR_OP_LAYERNORM_BWD, *shape, dtype=fr.FR_BF16, ws_bytes=1 << 40)
        assert p.form == fr.FR_FORM_SPLIT and p.splits == -(-shape[1] // 8192)
        compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, ws=team_ws(*shape)), what=f"split {shape}")
        compare(x, dy, None, mean, rstd, run_bwd(x, dy, None, mean, rstd, ws=team_ws(*shape)),
                what=f"split no gamma {shape}")
        compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, want_dg=False, ws=team_ws(*shape)),
                what=f"split dx only {shape}")
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)


@pytest.mark.parametrize("shape", [(300, 32768), (7, 20000), (5, 16392)])
def test_layernorm_backward_split_rows_recomputed_partner_sums(shape):
    # with no wait every partner's row sums are recomputed by the waiting
    # workgroup: the same bits as the exchanged ones, and the workspace
    # header counts them (rows x parts x (parts - 1)); 4, 3 and 3 parts, the
    # last one narrower in the second and third shapes
    rows, cols = shape
    parts = -(-cols // 8192)
    x, dy, g, mean, rstd = inputs(rows, cols, seed=23)
    ws = team_ws(rows, cols)
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        n0 = recomputed(ws)
        a = run_bwd(x, dy, g, mean, rstd, ws=ws)
        # how many the default wait recomputed depends on scheduling: reported
        print(f"{shape}: {recomputed(ws) - n0} partner sums recomputed with the default wait")
        fr.fr_tune_override(fr.FR_OP_LAYERNORM_BWD, form=fr.FR_FORM_SPLIT, threads=1024, vec=1, wait_us=-1)
        try:
            n0 = recomputed(ws)
            b = run_bwd(x, dy, g, mean, rstd, ws=ws)
        finally:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM_BWD)
        assert recomputed(ws) - n0 == rows * parts * (parts - 1)
        # a 1 us wait: partner sums are read where they arrived in time and
        # recomputed where not (the counter says how many); the same bits
        fr.fr_tune_override(fr.FR_OP_LAYERNORM_BWD, form=fr.FR_FORM_SPLIT, threads=1024, vec=1, wait_us=1)
        try:
            n0 = recomputed(ws)
            c = run_bwd(x, dy, g, mean, rstd, ws=ws)
        finally:
            fr.fr_tune_override(fr.FR_OP_LAYERNORM_BWD)
        assert 0 <= recomputed(ws) - n0 <= rows * parts * (parts - 1)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)
    for k in ("dx", "dgamma", "dbeta"):
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k
    compare(x, dy, g, mean, rstd, a, what=f"split {shape}")


@pytest.mark.parametrize("kind", ["garbage", "softmax-initialized"])
def test_layernorm_backward_split_rows_untrusted_workspace(kind):
    """A workspace the backward's init has not prepared - random words, or
    one prepared for the split softmax (another mark) - has no slot trusted:
    every partner's sums are recomputed, with the bits of an initialized
    workspace, and the results match the oracle."""
    rows, cols = 40, 24576
    parts = 3
    x, dy, g, mean, rstd = inputs(rows, cols, seed=31)
    good = team_ws(rows, cols)
    bad = team_ws(rows, cols, init=False)
    if kind == "garbage":
        gen = torch.Generator(device="cuda")
        gen.manual_seed(37)
        bad.view(torch.int32).copy_(torch.randint(-2**31, 2**31 - 1, bad.shape, generator=gen, device="cuda",
                                                  dtype=torch.int32))
    else:
        fr.fr_softmax_rows_workspace_init(bad)
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        a = run_bwd(x, dy, g, mean, rstd, ws=good)
        n0 = recomputed(bad)
        b = run_bwd(x, dy, g, mean, rstd, ws=bad)
        assert (recomputed(bad) - n0) % (1 << 32) == rows * parts * (parts - 1)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)
    for k in ("dx", "dgamma", "dbeta"):
        assert np.array_equal(a[k], b[k]), k
    compare(x, dy, g, mean, rstd, b, what=f"{kind} workspace")


def test_layernorm_backward_persistent_call_leaves_no_trusted_slot():
    """A call that takes the persistent form writes its partial rows into
    the bytes the split form's slots use, and clears the workspace's mark:
    a split call that follows trusts no slot (every partner's sums
    recomputed, the same bits), until the workspace is initialized again."""
    rows, cols = 48, 32768
    parts = 4
    x, dy, g, mean, rstd = inputs(rows, cols, seed=47)
    ws = team_ws(rows, cols)
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        a = run_bwd(x, dy, g, mean, rstd, ws=ws)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)
    # in place: the persistent form, same workspace
    b = run_bwd(x, dy, g, mean, rstd, ws=ws, inplace=True)
    compare(x, dy, g, mean, rstd, b, what="persistent, in place")
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        n0 = recomputed(ws)
        c = run_bwd(x, dy, g, mean, rstd, ws=ws)
        assert (recomputed(ws) - n0) % (1 << 32) == rows * parts * (parts - 1)
        fr.fr_layernorm_rows_backward_workspace_init(ws)
        n0 = recomputed(ws)
        d = run_bwd(x, dy, g, mean, rstd, ws=ws)
        assert recomputed(ws) - n0 <= rows * parts * (parts - 1)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)
    for k in ("dx", "dgamma", "dbeta"):
        assert np.array_equal(a[k], c[k]), k
        assert np.array_equal(a[k], d[k]), k


def test_layernorm_backward_split_rows_workspace_reused_across_calls():
    """Calls that share one workspace, with different inputs in between,
    never read an earlier call's sums: every call matches the oracle, and
    repeats give the same bits."""
    rows, cols = 64, 32768
    ws = team_ws(rows, cols)
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        outs = {}
        for it, seed in enumerate((41, 43, 41, 43, 41)):
            x, dy, g, mean, rstd = inputs(rows, cols, seed=seed)
            r = run_bwd(x, dy, g, mean, rstd, ws=ws)
            if seed in outs:
                for k in ("dx", "dgamma", "dbeta"):
                    assert np.array_equal(outs[seed][k], r[k]), (it, k)
            else:
                outs[seed] = r
                compare(x, dy, g, mean, rstd, r, what=f"call {it} seed {seed}")
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)


def test_layernorm_backward_split_rows_choice_and_errors():
    rows, cols = 256, 16384
    x, dy, g, mean, rstd = inputs(rows, cols, seed=29)
    ws = team_ws(rows, cols)
    # automatic: split rows with a workspace and 16-byte accesses ...
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM_BWD, rows, cols, dtype=fr.FR_BF16, ws_bytes=ws.numel() * 4)
    assert (p.form, p.splits, p.chunk, p.grid) == (fr.FR_FORM_SPLIT, 2, 8192, 256)
    a = run_bwd(x, dy, g, mean, rstd, ws=ws)
    compare(x, dy, g, mean, rstd, a, what="auto split")
    # ... persistent rows when dx overwrites an input, with the same workspace
    b = run_bwd(x, dy, g, mean, rstd, ws=ws, inplace=True)
    compare(x, dy, g, mean, rstd, b, what="in place")
    # persistent rows without a workspace (dx only)
    compare(x, dy, g, mean, rstd, run_bwd(x, dy, g, mean, rstd, want_dg=False), what="dx only, no workspace")
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        with pytest.raises(fr.FrError) as ei:  # split rows never write over x or dy
            run_bwd(x, dy, g, mean, rstd, ws=ws, inplace=True)
        assert ei.value.status == fr.FR_E_ARG
        with pytest.raises(fr.FrError) as ei:  # the exchange slots need a workspace
            run_bwd(x, dy, g, mean, rstd, want_dg=False)
        assert ei.value.status == fr.FR_E_WORKSPACE
        with pytest.raises(fr.FrError) as ei:  # 16-byte accesses only
            run_bwd(x, dy, g, mean, rstd, offset=1, ws=ws)
        assert ei.value.status == fr.FR_E_ARG
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)


def test_layernorm_backward_split_rows_deterministic():
    rows, cols = 2048, 32768
    x, dy, g, mean, rstd = inputs(rows, cols, seed=31)
    ws = team_ws(rows, cols)
    a = run_bwd(x, dy, g, mean, rstd, ws=ws)
    b = run_bwd(x, dy, g, mean, rstd, ws=ws)
    for k in ("dx", "dgamma", "dbeta"):
        assert np.array_equal(a[k], b[k]), k


def test_layernorm_backward_split_rows_graph_replays():
    # the reset of the exchange slots is a fill kernel, so the call can be
    # recorded in a graph: every replay (with eager calls on other data and
    # synchronisations between them) equals the eager result bit for bit
    rows, cols = 512, 32768
    x, dy, g, mean, rstd = inputs(rows, cols, seed=37)
    x2, dy2, _, mean2, rstd2 = inputs(rows, cols, seed=41)
    xd, dyd, gd, md, rd = bf16_bits_tensor(x), bf16_bits_tensor(dy), bf16_bits_tensor(g), dev(mean), dev(rstd)
    x2d, dy2d, m2d, r2d = bf16_bits_tensor(x2), bf16_bits_tensor(dy2), dev(mean2), dev(rstd2)
    ws = team_ws(rows, cols)
    dx = torch.empty_like(xd)
    dg = torch.empty(cols, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)
    dx2, dg2, db2 = torch.empty_like(dx), torch.empty_like(dg), torch.empty_like(db)

    def call():
        fr.fr_layernorm_rows_backward(xd, dyd, md, rd, dx, gamma=gd, dgamma=dg, dbeta=db, ws=ws)

    call()
    torch.cuda.synchronize()
    ref = (bf16_bits_of(dx), host(dg), host(db))
    compare(x, dy, g, mean, rstd, {"dx": ref[0], "dgamma": ref[1], "dbeta": ref[2]}, what="eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        dx.fill_(0)
        dg.fill_(float("nan"))
        # eager work on other data through the same workspace
        fr.fr_layernorm_rows_backward(x2d, dy2d, m2d, r2d, dx2, gamma=gd, dgamma=dg2, dbeta=db2, ws=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_of(dx), ref[0]), rep
        assert np.array_equal(host(dg), ref[1]) and np.array_equal(host(db), ref[2]), rep
