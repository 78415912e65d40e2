"""Host-side tests of libfr (no GPU needed).

The C ABI library must load, export every symbol include/fr.h declares,
reject invalid arguments with the documented status before any HIP call, and
plan the expected reduction form and launch configuration for the five
workloads. No compute call is made here.
"""
import ctypes
import os
import re

import pytest

import pointwise_reduction_amd as fr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "fr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fr_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = header_functions()
    assert set(declared) == set(fr.EXPORTS)
    for name in declared:
        assert hasattr(fr.lib, name), name


def test_status_strings_and_version():
    assert fr.status_string(fr.FR_OK).startswith("FR_OK")
    for code in range(-1, -10, -1):
        assert fr.status_string(code).startswith("FR_E_")
    assert fr.status_string(12345) == "unknown status"
    assert fr.lib.fr_version() >= 100


# ------------------------------------------------------------------ validation (returns before any HIP call)

P = ctypes.c_void_p
FAKE = P(0x10000)  # never dereferenced: every call below fails validation first
FAKE_ODD = P(0x10002)


def softmax(x=FAKE, y=FAKE, rows=4, cols=8, x_rs=8, x_cs=1, y_rs=8, y_cs=1, lengths=None, argmax=None, ws=None,
            ws_bytes=0, dtype=fr.FR_F32):
    return fr.lib.fr_softmax_rows(x, y, rows, cols, x_rs, x_cs, y_rs, y_cs, lengths, argmax, ws, ws_bytes, dtype,
                                  None)


def test_softmax_argument_errors():
    assert softmax(rows=-1) == fr.FR_E_SIZE
    assert softmax(cols=1 << 30) == fr.FR_E_SIZE
    assert softmax(dtype=fr.FR_BF16) == fr.FR_E_DTYPE
    assert softmax(x=None) == fr.FR_E_NULL
    assert softmax(y=None) == fr.FR_E_NULL
    assert softmax(x_cs=2) == fr.FR_E_STRIDE
    assert softmax(y_rs=7) == fr.FR_E_STRIDE
    assert softmax(x_rs=-8) == fr.FR_E_STRIDE
    assert softmax(x=FAKE_ODD) == fr.FR_E_ALIGN
    assert softmax(y=FAKE, x=FAKE, y_rs=16) == fr.FR_E_STRIDE  # in place needs equal strides
    assert softmax(ws=P(0x10008), ws_bytes=1 << 20) == fr.FR_E_ALIGN
    assert softmax(cols=100000, x_rs=100000, y_rs=100000, ws=FAKE, ws_bytes=16) == fr.FR_E_WORKSPACE
    # empty work returns before touching anything
    assert softmax(rows=0, x=None, y=None) == fr.FR_OK
    assert softmax(cols=0, x=None, y=None) == fr.FR_OK


def test_sum_relu_add_argument_errors():
    f = fr.lib.fr_sum_relu_add
    ok = dict(a=FAKE, b=FAKE, out=FAKE, rows=4, cols=8, a_rs=8, a_cs=1, b_rs=8, b_cs=1, out_s=1, ws=None,
              ws_bytes=0, dtype=fr.FR_F32)

    def call(**kw):
        args = dict(ok, **kw)
        return f(args["a"], args["b"], args["out"], args["rows"], args["cols"], args["a_rs"], args["a_cs"],
                 args["b_rs"], args["b_cs"], args["out_s"], args["ws"], args["ws_bytes"], args["dtype"], None)

    assert call(rows=-3) == fr.FR_E_SIZE
    assert call(dtype=fr.FR_BF16) == fr.FR_E_DTYPE
    assert call(b=None) == fr.FR_E_NULL
    assert call(out=None) == fr.FR_E_NULL
    assert call(b_cs=0) == fr.FR_E_STRIDE
    assert call(a_rs=4) == fr.FR_E_STRIDE
    assert call(out_s=0) == fr.FR_E_STRIDE
    assert call(out=FAKE_ODD) == fr.FR_E_ALIGN
    assert call(rows=0, a=None, b=None, out=None) == fr.FR_OK


def test_layernorm_argument_errors():
    f = fr.lib.fr_layernorm_rows

    def call(x=FAKE, g=None, b=None, y=FAKE, rows=2, cols=16, x_rs=16, x_cs=1, y_rs=16, y_cs=1, eps=1e-5,
             dtype=fr.FR_BF16):
        return f(x, g, b, y, rows, cols, x_rs, x_cs, y_rs, y_cs, eps, dtype, None)

    assert call(dtype=fr.FR_F32) == fr.FR_E_DTYPE
    assert call(cols=0) == fr.FR_E_SIZE
    assert call(eps=-1.0) == fr.FR_E_ARG
    assert call(eps=float("nan")) == fr.FR_E_ARG
    assert call(eps=float("inf")) == fr.FR_E_ARG
    assert call(x=None) == fr.FR_E_NULL
    assert call(y_cs=3) == fr.FR_E_STRIDE
    assert call(x=P(0x10001)) == fr.FR_E_ALIGN
    assert call(g=P(0x10001)) == fr.FR_E_ALIGN
    assert call(rows=0, x=None, y=None) == fr.FR_OK


def test_sumsq_argument_errors():
    full = fr.lib.fr_sumsq_full
    n = 1 << 20
    need = fr.fr_sumsq_full_workspace_bytes(n)
    assert need > 0
    assert full(FAKE, -1, FAKE, None, 0, fr.FR_F32, None) == fr.FR_E_SIZE
    assert full(FAKE, n, FAKE, None, 0, fr.FR_BF16, None) == fr.FR_E_DTYPE
    assert full(FAKE, n, None, FAKE, need, fr.FR_F32, None) == fr.FR_E_NULL
    assert full(None, n, FAKE, FAKE, need, fr.FR_F32, None) == fr.FR_E_NULL
    assert full(FAKE, n, FAKE, None, 0, fr.FR_F32, None) == fr.FR_E_WORKSPACE
    assert full(FAKE, n, FAKE, FAKE, need - 4, fr.FR_F32, None) == fr.FR_E_WORKSPACE
    assert full(FAKE, n, FAKE, P(0x10004), need, fr.FR_F32, None) == fr.FR_E_ALIGN
    rows_f = fr.lib.fr_sumsq_rows
    assert rows_f(FAKE, FAKE, 4, 8, 8, 2, None, 0, fr.FR_F32, None) == fr.FR_E_STRIDE
    assert rows_f(FAKE, None, 4, 8, 8, 1, None, 0, fr.FR_F32, None) == fr.FR_E_NULL


def test_workspace_init_argument_errors():
    # both split workspaces: checked before any HIP call
    for init in (fr.lib.fr_softmax_rows_workspace_init, fr.lib.fr_layernorm_rows_backward_workspace_init):
        assert init(None, 4096, None) == fr.FR_E_NULL
        assert init(P(0x10008), 4096, None) == fr.FR_E_ALIGN
        assert init(FAKE, 8, None) == fr.FR_E_WORKSPACE


def test_layernorm_backward_team_header_holds_every_flag():
    # the split-row backward's grid never exceeds the flags its header holds
    # (256 workgroups): the largest team grids the planner makes
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        for rows, cols in ((100000, 32768), (4096, 8200), (300, 16392), (1 << 20, 24576), (1, 8200)):
            p = fr.fr_plan_query(fr.FR_OP_LAYERNORM_BWD, rows, cols, dtype=fr.FR_BF16, ws_bytes=1 << 40)
            assert p.form == fr.FR_FORM_SPLIT and p.grid <= 256 and p.grid % p.splits == 0, (rows, cols, p.grid)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)


def test_stream_reference_argument_errors():
    copy, read = fr.lib.fr_stream_copy, fr.lib.fr_stream_read
    assert copy(FAKE, P(0x20000), 17, None) == fr.FR_E_SIZE
    assert copy(FAKE, P(0x20000), -16, None) == fr.FR_E_SIZE
    assert copy(FAKE, None, 32, None) == fr.FR_E_NULL
    assert copy(P(0x10008), P(0x20000), 32, None) == fr.FR_E_ALIGN
    assert copy(P(0x10000), P(0x10010), 64, None) == fr.FR_E_ARG  # overlapping
    assert copy(None, None, 0, None) == fr.FR_OK  # nothing to move, no HIP call
    assert read(FAKE, 8, FAKE, None) == fr.FR_E_SIZE
    assert read(FAKE, 16, None, None) == fr.FR_E_NULL
    assert read(P(0x10004), 16, FAKE, None) == fr.FR_E_ALIGN
    write = fr.lib.fr_stream_write
    assert write(FAKE, 24, 0, None) == fr.FR_E_SIZE
    assert write(FAKE, -16, 0, None) == fr.FR_E_SIZE
    assert write(None, 16, 0, None) == fr.FR_E_NULL
    assert write(P(0x10008), 32, 0, None) == fr.FR_E_ALIGN
    assert write(None, 0, 0, None) == fr.FR_OK  # nothing to write, no HIP call


def test_attn_decode_argument_errors():
    f = fr.lib.fr_attn_decode
    ws_need = fr.fr_attn_decode_workspace_bytes(2, 8, 1000, 128)
    assert ws_need == 2 * 8 * 4 * (128 + 4) * 4  # 4 chunks of 256 keys, one (m, l, pad, pad, a) slot each

    def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, Hq=8, Hkv=2, S=1000, D=128, L=None, scale=0.1,
             ws=FAKE, wsb=ws_need, dt=fr.FR_BF16):
        return f(q, k, v, o, lse, B, Hq, Hkv, S, D, L, scale, ws, wsb, dt, None)
    assert call(dt=7) == fr.FR_E_DTYPE
    assert call(D=96) == fr.FR_E_SIZE
    assert call(S=-1) == fr.FR_E_SIZE
    assert call(B=70000) == fr.FR_E_SIZE
    assert call(Hkv=3) == fr.FR_E_ARG   # 8 query heads on 3 key-value heads
    assert call(Hq=32, Hkv=2) == fr.FR_E_ARG  # 16 query heads per key-value head
    assert call(scale=float("inf")) == fr.FR_E_ARG
    assert call(q=None) == fr.FR_E_NULL
    assert call(k=None) == fr.FR_E_NULL
    assert call(o=P(0x10008)) == fr.FR_E_ALIGN
    assert call(lse=P(0x10002)) == fr.FR_E_ALIGN
    assert call(wsb=ws_need - 1) == fr.FR_E_WORKSPACE
    assert call(ws=None) == fr.FR_E_WORKSPACE
    assert call(B=0) == fr.FR_OK and call(Hq=0) == fr.FR_OK  # nothing to compute, no HIP call
    assert fr.fr_attn_decode_workspace_bytes(2, 8, 1000, 80) == 0


def test_softmax_backward_argument_errors_and_plans():
    f = fr.lib.fr_softmax_rows_backward

    def call(y=FAKE, dy=FAKE, dx=P(0x20000), rows=4, cols=8, ys=(8, 1), gs=(8, 1), xs=(8, 1), L=None,
             dt=fr.FR_F32):
        return f(y, dy, dx, rows, cols, ys[0], ys[1], gs[0], gs[1], xs[0], xs[1], L, dt, None)
    assert call(dt=fr.FR_BF16) == fr.FR_E_DTYPE
    assert call(cols=-1) == fr.FR_E_SIZE
    assert call(y=None) == fr.FR_E_NULL
    assert call(gs=(8, 2)) == fr.FR_E_STRIDE
    assert call(dx=FAKE, xs=(16, 1)) == fr.FR_E_STRIDE  # dx aliases y with another row stride
    assert call(dx=FAKE_ODD) == fr.FR_E_ALIGN
    assert call(L=P(0x10002)) == fr.FR_E_ALIGN
    assert call(rows=0) == fr.FR_OK and call(cols=0) == fr.FR_OK  # nothing to do, no HIP call
    p = fr.fr_plan_query(fr.FR_OP_SOFTMAX_BWD, 4096, 1024)
    assert (p.form, p.seg, p.vec, p.rows_per_wg) == (fr.FR_FORM_PER, 64, 4, 4)
    p = fr.fr_plan_query(fr.FR_OP_SOFTMAX_BWD, 512, 50257)
    assert (p.form, p.threads, p.vec, p.grid) == (fr.FR_FORM_RED, 512, 2, 512)
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_SOFTMAX_BWD, 4, 1 << 20, ws_bytes=1 << 30)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)


# ------------------------------------------------------------------ planning


def test_plans_for_the_five_workloads():
    # Example 1.1, 64 x 128 fp32: half a wave per row, one vector per lane
    p = fr.fr_plan_query(fr.FR_OP_SUM_RELU_ADD, 64, 128)
    assert (p.form, p.seg, p.vec, p.rows_per_wg, p.grid) == (fr.FR_FORM_PER, 32, 1, 8, 8)
    # softmax 4096 x 1024: a wave per 2 rows, 4 x 16-byte vectors per lane and row
    p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024)
    assert (p.form, p.seg, p.vec, p.rows_per_wg, p.grid) == (fr.FR_FORM_PER, 64, 4, 8, 512)
    # LayerNorm 2048 x 32768 bf16: a 512-thread workgroup holds a row; one
    # workgroup per CU takes 8 rows with 3 in flight
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16)
    assert (p.form, p.threads, p.vec, p.rows_per_wg, p.grid) == (fr.FR_FORM_PER, 512, 8, 8, 256)
    # a workgroup per row below 3 rows per CU, for other row lengths, and for
    # rows without 16-byte alignment
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 767, 32768, dtype=fr.FR_BF16)
    assert (p.rows_per_wg, p.grid) == (1, 767)
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 768, 32768, dtype=fr.FR_BF16)
    assert (p.rows_per_wg, p.grid) == (3, 256)
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 1000, 32768, dtype=fr.FR_BF16, num_cus=304)
    assert (p.rows_per_wg, p.grid) == (4, 250)
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 65536, 32768, dtype=fr.FR_BF16)
    assert (p.rows_per_wg, p.grid) == (8, 8192)
    assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 16384, dtype=fr.FR_BF16).rows_per_wg == 1
    assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16, aligned16=False).rows_per_wg == 1
    # a tuner's override picks either form
    fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=512, vec=8, rows_per_wg=5)
    try:
        p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16)
        assert (p.rows_per_wg, p.grid) == (5, 410)
        fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=512, vec=8)
        assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16).grid == 2048
        fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=1024, vec=4, rows_per_wg=8)
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16)
    finally:
        fr.fr_tune_override(fr.FR_OP_LAYERNORM)
    # sum of squares over 2^28: 512 chunks of 2^19 plus a finishing pass
    n = 1 << 28
    ws = fr.fr_sumsq_full_workspace_bytes(n)
    assert ws == 512 * 4
    p = fr.fr_plan_query(fr.FR_OP_SUMSQ, 1, n, ws_bytes=ws)
    assert (p.form, p.splits, p.chunk, p.grid, p.grid2) == (fr.FR_FORM_SPLIT, 512, 1 << 19, 512, 1)
    # ragged softmax, 512 rows of capacity 131072, with a workspace: 16 chunks of 8192, a
    # 64-byte header, 4096 workgroup flags and 512 x 16 partial slots of 16 bytes; one kernel
    # whose grid is every workgroup that can be resident at once (4 per CU at 256 threads,
    # two chunks in registers), waiting 200 us by default
    ws = fr.fr_softmax_rows_workspace_bytes(512, 131072)
    assert ws == 64 + 4 * 4096 + 512 * 16 * 16
    p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, has_lengths=True, ws_bytes=ws)
    assert (p.form, p.splits, p.chunk, p.passes, p.grid, p.grid2, p.wait_us) == \
        (fr.FR_FORM_SPLIT, 16, 8192, 1, 256 * 4, 0, 200)
    # the two-kernel form (a tuning candidate) uses the same workspace
    fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=2)
    try:
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, has_lengths=True, ws_bytes=ws)
        assert (p.passes, p.grid, p.grid2, p.ws_bytes, p.wait_us) == (2, 8192, 8192, ws, 0)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
    # more rows than the single pass keeps in LDS: two kernels
    fr.fr_force_form(fr.FR_FORM_SPLIT)
    try:
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 3000, 131072, ws_bytes=1 << 30)
        assert (p.form, p.passes, p.grid) == (fr.FR_FORM_SPLIT, 2, 3000 * 16)
    finally:
        fr.fr_force_form(fr.FR_FORM_AUTO)
    # ... and without one: one workgroup streams each row
    p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, has_lengths=True)
    assert (p.form, p.threads, p.grid) == (fr.FR_FORM_RED, 512, 512)


def test_plan_thresholds_and_forms():
    # persistent up to 2048 fp32 per row, then looped
    assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 100, 2048).form == fr.FR_FORM_PER
    assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 100, 2049).form == fr.FR_FORM_RED
    # lane-group sizes follow the row length; masked tails round up
    assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 1, 1).seg == 8
    assert (fr.fr_plan_query(fr.FR_OP_SOFTMAX, 256, 1000).seg, fr.fr_plan_query(fr.FR_OP_SOFTMAX, 256, 1000).vec) == (64, 4)
    assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 1, 65).seg == 32
    # many long rows: looped even with a workspace; few long rows: split
    ws = fr.fr_sum_workspace_bytes(4096, 65536)
    assert fr.fr_plan_query(fr.FR_OP_SUMSQ, 4096, 65536, ws_bytes=ws).form == fr.FR_FORM_RED
    ws = fr.fr_sum_workspace_bytes(64, 16384)
    p = fr.fr_plan_query(fr.FR_OP_SUMSQ, 64, 16384, ws_bytes=ws)
    assert p.form == fr.FR_FORM_SPLIT and p.splits * p.chunk >= 16384 and p.ws_bytes == ws
    # unaligned bf16 rows use element accesses and smaller register tiles
    p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 4, 16384, dtype=fr.FR_BF16, aligned16=False)
    assert (p.form, p.vec16, p.vec) == (fr.FR_FORM_PER, 0, 4)
    assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, 4, 16385, dtype=fr.FR_BF16, aligned16=False).form == fr.FR_FORM_RED
    assert fr.fr_plan_query(fr.FR_OP_LAYERNORM, 4, 32769, dtype=fr.FR_BF16).form == fr.FR_FORM_RED


def test_forced_forms():
    prev = fr.fr_force_form(fr.FR_FORM_RED)
    try:
        assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 7, 13).form == fr.FR_FORM_RED
        fr.fr_force_form(fr.FR_FORM_SPLIT)
        with pytest.raises(fr.FrError) as e:
            fr.fr_plan_query(fr.FR_OP_SOFTMAX, 7, 13)  # no workspace
        assert e.value.status == fr.FR_E_ARG
        ws = fr.fr_softmax_rows_workspace_bytes(7, 13)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 7, 13, ws_bytes=ws)
        assert (p.form, p.splits) == (fr.FR_FORM_SPLIT, 1)
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_LAYERNORM, 7, 13, dtype=fr.FR_BF16)  # LayerNorm rows never split
        fr.fr_force_form(fr.FR_FORM_PER)
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_SOFTMAX, 7, 4096)  # too long for registers
    finally:
        fr.fr_force_form(prev)
    assert fr.fr_force_form(fr.FR_FORM_AUTO) == prev


def test_workspace_matches_example_6_2_layout(golden):
    # Example 6.2 keeps 2 fp32 partials per row for 64 rows (512 bytes). Our
    # plan for the same shape keeps more partials per row (more workgroups
    # for 256 CUs), still one fp32 per (row, chunk).
    g = golden("stax4_example_6_2.txt")
    rows, cols = int(g["rows"]), int(g["cols"])
    p = fr.fr_plan_query(fr.FR_OP_SUMSQ, rows, cols, ws_bytes=1 << 20)
    assert p.form == fr.FR_FORM_SPLIT
    assert p.ws_bytes == rows * p.splits * 4
    assert p.splits >= g["splits"]
    assert fr.fr_sum_workspace_bytes(rows, cols) == p.ws_bytes


def test_tune_override_replaces_the_launch_knobs():
    try:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_PER, threads=256, seg=64, vec=4, rows_per_wg=4)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024)
        assert (p.form, p.seg, p.vec, p.rows_per_wg, p.grid) == (fr.FR_FORM_PER, 64, 4, 4, 1024)
        with pytest.raises(fr.FrError) as e:
            fr.fr_plan_query(fr.FR_OP_SOFTMAX, 10, 4000)  # does not fit 64 lanes x 4 vectors
        assert e.value.status == fr.FR_E_ARG
        # a split candidate with smaller chunks needs more workspace than the default query gives
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=4)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, ws_bytes=1 << 30)
        assert (p.splits, p.chunk, p.passes) == (32, 4096, 1)
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=8, passes=2)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, ws_bytes=1 << 30)
        assert (p.splits, p.passes, p.grid, p.grid2, p.ws_bytes) == (16, 2, 8192, 8192, 64 + 4 * 4096 + 512 * 16 * 16)
        # the single pass with 512 threads: 2 resident workgroups per CU; wait overrides pass through
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=512, vec=4, passes=1, wait_us=-1)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, ws_bytes=1 << 30)
        assert (p.splits, p.passes, p.grid, p.wait_us) == (16, 1, 512, -1)
        # more rows than the single pass keeps in LDS
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_SOFTMAX, 2049, 65 * 8192, ws_bytes=1 << 40)
        fr.fr_tune_override(fr.FR_OP_SOFTMAX, form=fr.FR_FORM_SPLIT, threads=256, vec=4)
        with pytest.raises(fr.FrError) as e:
            fr.fr_plan_query(fr.FR_OP_SOFTMAX, 512, 131072, ws_bytes=fr.fr_softmax_rows_workspace_bytes(512, 131072))
        assert e.value.status == fr.FR_E_WORKSPACE  # 32 chunks per row need twice the default partials
        fr.fr_tune_override(fr.FR_OP_LAYERNORM, form=fr.FR_FORM_PER, threads=1024, vec=4)
        p = fr.fr_plan_query(fr.FR_OP_LAYERNORM, 2048, 32768, dtype=fr.FR_BF16)
        assert (p.threads, p.vec, p.occupancy) == (1024, 4, 0)
    finally:
        fr.fr_tune_override(fr.FR_OP_SOFTMAX)
        fr.fr_tune_override(fr.FR_OP_LAYERNORM)
    assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024).rows_per_wg == 8  # automatic: 2 rows per wave
    with pytest.raises(fr.FrError):
        fr.fr_tune_override(99, form=1)


def test_pointwise_plans_and_argument_errors():
    p = fr.fr_plan_query(fr.FR_OP_ADD_2D, 8192, 8192)
    assert (p.form, p.rows_per_wg, p.chunk, p.grid) == (fr.FR_FORM_POINTWISE, 64, 128, 128 * 64)
    p = fr.fr_plan_query(fr.FR_OP_ADD_2D, 0, 5)
    assert p.grid == 0
    with pytest.raises(fr.FrError):
        fr.fr_plan_query(fr.FR_OP_ADD_2D, 4, 4, dtype=fr.FR_BF16)
    p = fr.fr_plan_query(fr.FR_OP_GELU_BWD, 1, 1 << 28)
    assert (p.form, p.vec, p.grid) == (fr.FR_FORM_POINTWISE, 2, (1 << 26) // 512)
    p = fr.fr_plan_query(fr.FR_OP_GELU_BWD, 1, 1000, dtype=fr.FR_BF16, aligned16=False)
    assert p.grid == 4  # element accesses: 256 per workgroup step
    prev = fr.fr_force_form(fr.FR_FORM_PER)
    try:
        with pytest.raises(fr.FrError):
            fr.fr_plan_query(fr.FR_OP_ADD_2D, 64, 64)
    finally:
        fr.fr_force_form(prev)
    fr.fr_tune_override(fr.FR_OP_ADD_2D, form=fr.FR_FORM_POINTWISE, threads=256, rows_per_wg=32, chunk=100)
    try:
        with pytest.raises(fr.FrError):  # 32 x 100 is not a whole number of 1024-element passes
            fr.fr_plan_query(fr.FR_OP_ADD_2D, 64, 64)
    finally:
        fr.fr_tune_override(fr.FR_OP_ADD_2D)
    # arguments rejected before any HIP call (no GPU needed)
    assert fr.lib.fr_add_2d(None, 4, 1, None, 4, 1, None, 4, 2, 4, fr.FR_F32, None) == fr.FR_E_NULL
    assert fr.lib.fr_add_2d(None, 4, 1, None, 4, 1, None, 4, 0, 4, fr.FR_F32, None) == fr.FR_OK
    assert fr.lib.fr_add_2d(None, 4, 1, None, 4, 1, None, 4, 2, 4, fr.FR_BF16, None) == fr.FR_E_DTYPE
    assert fr.lib.fr_gelu_backward(None, 2, None, None, 8, fr.FR_F32, None) == fr.FR_E_STRIDE
    assert fr.lib.fr_gelu_backward(None, 0, None, None, 0, fr.FR_F32, None) == fr.FR_OK
    assert fr.lib.fr_gelu_backward(None, 0, None, None, -1, fr.FR_F32, None) == fr.FR_E_SIZE


def test_region_object_without_a_gpu():
    # create / state / counts / destroy and the argument checks make no HIP call
    r = fr.Region()
    assert r.state == fr.FR_REGION_EMPTY and r.counts() == (0, 0)
    assert fr.lib.fr_region_run(r._r, None, 0, None, None, None) == fr.FR_E_NULL
    assert fr.lib.fr_region_run(r._r, None, 8, fr._REGION_FN(lambda c, s: 0), None, None) == fr.FR_E_NULL
    assert fr.lib.fr_region_state(None) == fr.FR_E_NULL
    del r


def test_build_rejects_a_single_pass_kernel_below_the_occupancy_its_grid_assumes():
    from pointwise_reduction_amd import build as b
    name = "_ZN2fr20fr_split_softmax_oneILi256ELi8ELb1EEEvPKfPf"
    b.check_residency({name: {"occupancy": 4, "vgpr": 111}})
    with pytest.raises(RuntimeError, match="waves per SIMD"):
        b.check_residency({name: {"occupancy": 3, "vgpr": 131}})
