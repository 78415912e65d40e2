"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only. Each test ties an oracle function to something other than itself:
values printed on the pages (tests/golden), closed forms, invariants, exact
rational brute force on tiny inputs, or library routines (scipy, torch,
math.fsum) for the special cases that reduce to them. They are chosen so that
a dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import synth

# ------------------------------------------------------------ Example 1.1 (C1)


def test_sum_relu_add_tiny_by_hand():
    # 2*(relu(1.5) + relu(-1) + relu(-0.5)) = 3
    a = np.array([[1.0, -2.0, 0.5]], dtype=np.float32)
    b = np.array([[0.5, 1.0, -1.0]], dtype=np.float32)
    out, out64 = oracle.sum_relu_add(a, b)
    assert out[0] == 3.0 and out64[0] == 3.0


def test_sum_relu_add_closed_forms():
    R = 128
    c = np.float32(0.25)
    a = np.full((4, R), c, dtype=np.float32)
    out, _ = oracle.sum_relu_add(a, a)
    assert np.all(out == 4 * c * R)  # 2 * (2c) * R
    u = synth.uniform((8, R), seed=11)
    out, _ = oracle.sum_relu_add(u, -u)
    assert np.all(out == 0.0)
    neg = -np.abs(synth.uniform((8, R), seed=12)) - np.float32(0.01)
    out, _ = oracle.sum_relu_add(neg, neg)
    assert np.all(out == 0.0)


def test_sum_relu_add_exact_grid_brute_force():
    # entries on {-1,-1/2,0,1/2,1}: brute force in exact rationals
    rng = np.random.default_rng(5)
    grid = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32)
    a = grid[rng.integers(0, 5, size=(16, 37))]
    b = grid[rng.integers(0, 5, size=(16, 37))]
    out, _ = oracle.sum_relu_add(a, b)
    for i in range(16):
        s = sum(2 * max(Fraction(float(a[i, r])) + Fraction(float(b[i, r])), Fraction(0)) for r in range(37))
        assert Fraction(float(out[i])) == s


def test_sum_relu_add_matches_example_10_1_expression():
    # Example 10.1 writes the operation as (relu(x + w) * 2).sum(-1); torch's
    # fp32 add then an fp64 sum is the same definition as a library routine.
    torch = pytest.importorskip("torch")
    a, b, _ = synth.sum_relu_add_inputs(64, 128, seed=1001)
    b = b[:, ::-1].copy()  # break any symmetry between the operands
    out, out64 = oracle.sum_relu_add(a, b)
    ref = (torch.relu(torch.from_numpy(a) + torch.from_numpy(b)).double() * 2).sum(-1).numpy()
    np.testing.assert_allclose(out64, ref, rtol=1e-13, atol=0)


def test_sum_relu_add_row_stride():
    a, b, _ = synth.sum_relu_add_inputs(8, 40, seed=3)
    big = np.zeros((8, 64), dtype=np.float32)
    big[:, :40] = a
    big[:, 40:] = 1e6  # must never be read
    out_view, _ = oracle.sum_relu_add(big[:, :40], b)
    out, _ = oracle.sum_relu_add(a, b)
    assert np.array_equal(out_view, out)


def test_sum_relu_add_nan_propagates_to_exactly_the_nan_rows():
    a, b, nan_rows = synth.sum_relu_add_inputs(64, 128, seed=1002, n_nan=4)
    assert len(nan_rows) == 4
    out, _ = oracle.sum_relu_add(a, b)
    assert set(np.nonzero(np.isnan(out))[0].tolist()) == set(nan_rows.tolist())


def test_sum_relu_add_inf_rules():
    inf = np.float32(np.inf)
    a = np.array([[inf, 1.0], [inf, 1.0], [-inf, 1.0]], dtype=np.float32)
    b = np.array([[-inf, 1.0], [1.0, 1.0], [1.0, 1.0]], dtype=np.float32)
    out, _ = oracle.sum_relu_add(a, b)
    assert math.isnan(out[0])  # inf + -inf = NaN, propagated by relu
    assert out[1] == np.inf
    assert out[2] == 4.0  # relu(-inf) = 0


# ------------------------------------------------------------ softmax (C2, C5)


def test_worked_example_probabilities(golden):
    g = golden("hello_gpu_ch12_worked_example.txt")
    tol = g["tolerance"]
    p = oracle.softmax_f64(g["scores"])
    np.testing.assert_allclose(p, g["probabilities"], atol=tol, rtol=0)
    m, d = oracle.md_fold(g["scores"])
    assert m == 4.0
    assert abs(d - g["exp_sum"]) < tol
    np.testing.assert_allclose(p * d, g["shifted_exps"], atol=tol, rtol=0)
    # the fp32-row entry point gives the same values
    y64, am = oracle.softmax_rows(np.array([g["scores"]], dtype=np.float32))
    np.testing.assert_allclose(y64[0], p, rtol=1e-15)
    assert am[0] == 2


def test_worked_example_weighted_output(golden):
    g = golden("hello_gpu_ch12_worked_example.txt")
    V = np.array(g["values"])
    p = oracle.softmax_f64(g["scores"])
    two_pass = p @ V
    np.testing.assert_allclose(two_pass, g["output"], atol=g["tolerance"], rtol=0)
    _, _, _, o = oracle.online_attention_row(g["scores"], V)
    np.testing.assert_allclose(o, two_pass, rtol=1e-14)


def test_online_trace_matches_figure_12_2(golden):
    g = golden("hello_gpu_ch12_worked_example.txt")
    tol = g["tolerance"]
    s = np.array(g["scores"])
    V = np.array(g["values"])
    m2, l2, a2, _ = oracle.online_attention_row(s[:2], V[:2])
    assert m2 == g["after_2_m"]
    assert abs(l2 - g["after_2_l"]) < tol
    np.testing.assert_allclose(a2, g["after_2_a"], atol=tol, rtol=0)
    m3, l3, a3, _ = oracle.online_attention_row(s, V)
    assert abs(math.exp(m2 - m3) - g["after_3_alpha"]) < tol
    assert abs(l3 - g["after_3_l"]) < tol
    np.testing.assert_allclose(a3, g["after_3_a"], atol=tol, rtol=0)
    # the page truncated a[1]: exact value 1 * e^-2 * 2e^-1... = 2 e^-3 + 1
    assert abs(a3[1] - (2 * math.exp(-3) + 1)) < 1e-15


def test_online_state_equals_two_pass_on_random_rows():
    rng = np.random.default_rng(7)
    for n in (1, 2, 3, 17, 300):
        s = rng.normal(size=n) * 5
        V = rng.normal(size=(n, 4))
        m, l, a, o = oracle.online_attention_row(s, V)
        assert m == s.max()
        assert abs(l - math.fsum(np.exp(s - s.max()))) <= 1e-13 * l
        np.testing.assert_allclose(o, oracle.softmax_f64(s) @ V, rtol=1e-12, atol=1e-15)


def _fold_segments(xs, cuts):
    parts = np.split(np.asarray(xs, dtype=np.float64), cuts)
    m, d = -math.inf, 0.0
    for part in parts:
        pm, pd = oracle.md_fold(part)
        m, d = oracle.md_combine(m, d, pm, pd)
    return m, d


def test_prop_9_1_every_order_and_segmentation():
    x = [2.0, 1.0, 4.0]
    ref = (4.0, math.exp(-2) + math.exp(-3) + 1.0)
    for perm in itertools.permutations(x):
        for k in range(0, 3):
            for cuts in itertools.combinations([1, 2], k):
                m, d = _fold_segments(perm, list(cuts))
                assert m == ref[0]
                assert abs(d - ref[1]) <= 2 * np.spacing(ref[1])


def test_md_monoid_identity_and_random_segmentation():
    assert oracle.md_combine(-math.inf, 0.0, -math.inf, 0.0) == (-math.inf, 0.0)
    assert oracle.md_combine(-math.inf, 0.0, 3.5, 1.0) == (3.5, 1.0)
    assert oracle.md_combine(3.5, 1.0, -math.inf, 0.0) == (3.5, 1.0)
    rng = np.random.default_rng(9)
    x = rng.normal(size=1000) * 4
    exact = math.fsum(np.exp(x - x.max()))
    for _ in range(5):
        cuts = sorted(rng.choice(np.arange(1, 1000), size=rng.integers(1, 30), replace=False).tolist())
        m, d = _fold_segments(rng.permutation(x), cuts)
        assert m == x.max()
        assert abs(d - exact) <= 1e-12 * exact


def test_softmax_rows_match_scipy():
    special = pytest.importorskip("scipy.special")
    x = synth.softmax_inputs(64, 1000, seed=2001)
    y64, am = oracle.softmax_rows(x)
    np.testing.assert_allclose(y64, special.softmax(x.astype(np.float64), axis=1), rtol=1e-13, atol=1e-300)
    assert np.array_equal(am, np.argmax(x, axis=1))


def test_softmax_closed_forms():
    for n in (1, 2, 3, 1000, 1024, 4097):
        y64, am = oracle.softmax_rows(np.full((1, n), 0.37, dtype=np.float32))
        assert np.all(np.float32(y64) == np.float32(1.0) / np.float32(n))
        assert am[0] == 0
    x = synth.softmax_inputs(4, 781, seed=3)
    y64, _ = oracle.softmax_rows(x)
    assert np.allclose(y64.sum(axis=1), 1.0, rtol=1e-14)
    # shift invariance with an exact shift (grid inputs, shift of 8)
    g = np.round(x * 4) / 4
    y1, _ = oracle.softmax_rows(g.astype(np.float32))
    y2, _ = oracle.softmax_rows((g + 8).astype(np.float32))
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    # permutation invariance
    perm = np.random.default_rng(1).permutation(781)
    y3, _ = oracle.softmax_rows(np.ascontiguousarray(x[:, perm]))
    np.testing.assert_allclose(y3, y64[:, perm], rtol=1e-13)


def test_argmax_first_occurrence_and_nan_reading():
    x = np.array([[1, 5, 5, 2], [7, 7, 7, 7], [0, 1, np.nan, 9], [-3, np.nan, np.nan, 0]], dtype=np.float32)
    y64, am = oracle.softmax_rows(x)
    assert am.tolist() == [1, 0, 2, 1]
    assert np.all(np.isnan(y64[2])) and np.all(np.isnan(y64[3]))
    assert np.all(np.isfinite(y64[:2]))


def test_ragged_rows_read_and_write_only_the_prefix():
    x, L = synth.ragged_softmax_inputs(8, 4096, seed=21, choices=(1, 7, 1000, 4095))
    assert np.isnan(x[0, L[0]:]).all()  # tails hold NaN
    y64, am = oracle.softmax_rows(x, lengths=L)
    for r in range(8):
        n = L[r]
        assert np.all(np.isfinite(y64[r, :n])) and np.all(np.isnan(y64[r, n:]))
        np.testing.assert_allclose(y64[r, :n], oracle.softmax_f64(x[r, :n]), rtol=1e-15)
        assert am[r] == np.argmax(x[r, :n])
    y0, am0 = oracle.softmax_rows(x[:2], lengths=np.array([0, -5], dtype=np.int32))
    assert am0.tolist() == [-1, -1] and np.isnan(y0).all()


# ------------------------------------------------------------ LayerNorm (C3)


def test_bf16_rounding_known_values():
    assert oracle.f64_to_bf16(1.0) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 2.0**-8) == 0x3F80  # tie -> even
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0**-8) == 0x3F82  # tie -> even (up)
    assert oracle.f64_to_bf16(1.0 + 2.0**-8 + 2.0**-30) == 0x3F81  # above the tie
    assert oracle.f64_to_bf16(-2.0) == 0xC000
    assert oracle.f64_to_bf16(0.0) == 0 and oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(math.inf) == 0x7F80 and oracle.f64_to_bf16(-math.inf) == 0xFF80
    assert oracle.f64_to_bf16(math.nan) & 0x7FC0 == 0x7FC0
    assert oracle.f64_to_bf16(3.4e38) == 0x7F80 and oracle.f64_to_bf16(3.389e38) == 0x7F7F
    assert oracle.f64_to_bf16(math.ldexp(2 - 2.0**-8, 127)) == 0x7F80  # tie above the max -> even = inf
    assert oracle.f64_to_bf16(2.0**-133) == 0x0001  # smallest subnormal
    assert oracle.f64_to_bf16(2.0**-134) == 0x0000  # tie -> even (0)
    for h in (0x0001, 0x3F80, 0x7F7F, 0x8123, 0x4049):
        assert oracle.f64_to_bf16(oracle.bf16_to_f64(h)) == h


def test_bf16_rounding_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_layernorm_textbook_row():
    x = synth.to_bf16(np.array([[1, 2, 3, 4]], dtype=np.float32))
    _, y64, _ = oracle.layernorm_rows(x, eps=0.0)
    np.testing.assert_allclose(y64[0], [-1.34164, -0.44721, 0.44721, 1.34164], atol=1e-5)
    _, y64e, _ = oracle.layernorm_rows(x, eps=1e-5)
    np.testing.assert_allclose(y64e[0], (np.arange(1, 5) - 2.5) / math.sqrt(1.25 + 1e-5), rtol=1e-15)


def test_layernorm_constant_row_gives_beta_exactly():
    x, g, b = synth.layernorm_inputs(3, 4096, seed=31)
    x[:] = synth.to_bf16(np.full((3, 4096), 1.6875, dtype=np.float32))
    y, y64, _ = oracle.layernorm_rows(x, g, b)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))


def test_layernorm_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    x, g, b = synth.layernorm_inputs(16, 3000, seed=3001)
    y, y64, mag = oracle.layernorm_rows(x, g, b, eps=1e-5)
    xf = torch.from_numpy(synth.bf16_to_f32(x)).double()
    gf = torch.from_numpy(synth.bf16_to_f32(g)).double()
    bf = torch.from_numpy(synth.bf16_to_f32(b)).double()
    ref = torch.nn.functional.layer_norm(xf, (3000,), gf, bf, eps=1e-5).numpy()
    np.testing.assert_allclose(y64, ref, rtol=1e-12, atol=1e-13)
    assert np.all(mag >= np.abs(y64) - 1e-12)
    ref_bits = torch.from_numpy(ref).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # single fp64 rounding vs torch's fp64->fp32->bf16: equal or adjacent
    diff = np.abs(y.astype(np.int32) - ref_bits.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.999


def test_layernorm_moments_and_affine_invariance():
    x, _, _ = synth.layernorm_inputs(4, 2048, seed=33)
    _, y64, _ = oracle.layernorm_rows(x, eps=1e-5)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    var = xf.var(axis=1)
    assert np.all(np.abs(y64.mean(axis=1)) < 1e-12)
    np.testing.assert_allclose(y64.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # LN(2x + 1) == LN(x) with eps = 0: on a 1/8 grid within +/-15 both x and
    # 2x + 1 are exact in bf16 (at most 8 significant bits)
    xg = np.clip(np.round(xf * 8) / 8, -15, 15)
    x0 = synth.to_bf16(xg.astype(np.float32))
    xs = synth.to_bf16((xg * 2 + 1).astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(xs).astype(np.float64), xg * 2 + 1)
    _, y64s, _ = oracle.layernorm_rows(xs, eps=0.0)
    _, y640, _ = oracle.layernorm_rows(x0, eps=0.0)
    np.testing.assert_allclose(y64s, y640, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ sum of squares (C4)


def test_sumsq_closed_forms():
    assert oracle.sumsq(np.ones(1 << 20, dtype=np.float32)) == float(1 << 20)
    assert oracle.sumsq(np.arange(10, dtype=np.float32)) == 285.0
    n = 4096
    assert oracle.sumsq(np.arange(n, dtype=np.float32)) == (n - 1) * n * (2 * n - 1) // 6
    assert oracle.sumsq(np.zeros(0, dtype=np.float32)) == 0.0


def test_sumsq_matches_fsum():
    x = synth.sumsq_inputs(1 << 18, seed=4001)
    exact = math.fsum((x.astype(np.float64)) ** 2)
    # sequential fp64 summation of n nonnegative terms: |error| <= (n-1) u sum
    assert abs(oracle.sumsq(x) - exact) <= (x.size - 1) * 2.0**-53 * exact
    assert abs(exact - (1 << 18) / 3) < 0.01 * (1 << 18) / 3  # E[x^2] = 1/3 (sanity)


def test_example_6_2_split_rows_and_l2_norm(golden):
    g = golden("stax4_example_6_2.txt")
    rows, cols, splits = int(g["rows"]), int(g["cols"]), int(g["splits"])
    assert int(g["partial_elems"]) * splits == cols
    assert rows * splits * 4 == g["workspace_bytes"]
    x = synth.uniform((rows, cols), seed=62)
    s = oracle.sumsq_rows(x)
    halves = [[math.fsum(x[r, k * 8192:(k + 1) * 8192].astype(np.float64) ** 2) for k in range(splits)]
              for r in range(rows)]
    np.testing.assert_allclose(s, [h0 + h1 for h0, h1 in halves], rtol=1e-13)
    # CMU 15-779 Lecture 8, Exercise 1: the row L2 norm is sqrt of this sum
    np.testing.assert_allclose(np.sqrt(s), np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-13)


# ------------------------------------------------------------------ attention decode


def _attn_np(q, k, v, lengths, scale):
    """Independent numpy statement of the same definition (matrix form)."""
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = S if lengths is None else int(np.clip(lengths[b], 0, S))
        if L == 0:
            continue
        for h in range(Hq):
            s = scale * (k[b, h // G, :L] @ q[b, h])
            o[b, h] = scipy.special.softmax(s) @ v[b, h // G, :L]
            lse[b, h] = scipy.special.logsumexp(s)
    return o, lse


def test_attn_decode_worked_example(golden):
    """[HG12] 12.1: scores [2, 1, 4] (q = [1, 0], keys [2,0], [1,0], [4,0],
    scale 1) with values [1,0], [0,2], [3,1] give o = [2.6456, 0.9278]; lse
    is log(e^2 + e^1 + e^4) and log of the page's exponent sum plus the max."""
    g = golden("hello_gpu_ch12_worked_example.txt")
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[s, 0.0] for s in g["scores"]]]])
    v = np.array([[g["values"]]])
    o, lse, mag, smag = oracle.attn_decode(q, k, v, scale=1.0)
    assert np.allclose(o[0, 0], g["output"], atol=g["tolerance"])
    assert lse[0, 0] == pytest.approx(np.log(np.exp(2) + np.exp(1) + np.exp(4)), rel=1e-15)
    assert lse[0, 0] == pytest.approx(4 + np.log(g["exp_sum"]), abs=g["tolerance"])
    assert np.allclose(mag[0, 0], o[0, 0])  # nonnegative values: the size of the terms is o itself
    assert smag[0, 0] == 4.0


def test_attn_decode_closed_forms():
    rng = np.random.default_rng(71)
    v = rng.normal(size=(1, 1, 5, 8))
    k = rng.normal(size=(1, 1, 5, 8))
    # one key: o is that value row, lse its score
    q = rng.normal(size=(1, 1, 8))
    o, lse, _, _ = oracle.attn_decode(q, k[:, :, :1], v[:, :, :1], scale=0.5)
    assert np.array_equal(o[0, 0], v[0, 0, 0])
    assert lse[0, 0] == pytest.approx(0.5 * float(q[0, 0] @ k[0, 0, 0]), rel=1e-14)
    # a zero query scores every key 0: uniform weights, o = mean of the rows, lse = log(n)
    o, lse, _, _ = oracle.attn_decode(np.zeros((1, 1, 8)), k, v)
    assert np.allclose(o[0, 0], v[0, 0].mean(axis=0), rtol=0, atol=1e-15)
    assert lse[0, 0] == pytest.approx(np.log(5), rel=1e-15)
    # adding one vector u to every key shifts every score by scale * q.u:
    # o unchanged, lse shifted by that amount
    u = rng.normal(size=8)
    o1, l1, _, _ = oracle.attn_decode(q, k, v, scale=0.3)
    o2, l2, _, _ = oracle.attn_decode(q, k + u, v, scale=0.3)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13)
    assert l2[0, 0] - l1[0, 0] == pytest.approx(0.3 * float(q[0, 0] @ u), abs=1e-13)


def test_attn_decode_matches_matrix_form_with_groups_and_lengths():
    """Grouped heads (query head h reads key-value head h // (Hq / Hkv)),
    per-batch lengths (0, partial, full, beyond S clamped), against an
    independent numpy + scipy statement of softmax(scale q K^T) V."""
    rng = np.random.default_rng(72)
    B, Hq, Hkv, S, D = 4, 6, 2, 37, 16
    q = rng.normal(size=(B, Hq, D))
    k = rng.normal(size=(B, Hkv, S, D)) * 2
    v = rng.normal(size=(B, Hkv, S, D))
    lengths = np.array([0, 11, S, S + 5], dtype=np.int32)
    o, lse, mag, _ = oracle.attn_decode(q, k, v, lengths=lengths)
    o_np, lse_np = _attn_np(q, k, v, lengths, 1 / np.sqrt(D))
    assert np.allclose(o, o_np, rtol=1e-12, atol=1e-13)
    assert np.array_equal(o[0], np.zeros((Hq, D))) and np.all(np.isneginf(lse[0]))
    assert np.allclose(lse[1:], lse_np[1:], rtol=1e-13)
    assert np.all(mag >= np.abs(o) - 1e-15)
    # a mistake in the head mapping shows: swapping the key-value heads changes the result
    o_sw, _, _, _ = oracle.attn_decode(q, k[:, ::-1], v[:, ::-1], lengths=lengths)
    assert not np.allclose(o_sw[1:], o[1:])


def test_attn_merge_any_split_equals_the_whole():
    """[Stax4] 9.10: the (m, l, a) triples of any segmentation of the keys,
    merged with (+), give the triple of the whole row; o = a / l."""
    rng = np.random.default_rng(73)
    n, D = 23, 4
    s = rng.normal(size=n) * 3
    V = rng.normal(size=(n, D))
    m_all, l_all, a_all, o_all = oracle.online_attention_row(s, V)
    ident = (-np.inf, 0.0, np.zeros(D))
    for cut in range(0, n + 1):
        parts = [oracle.online_attention_row(s[:cut], V[:cut])[:3] if cut else ident,
                 oracle.online_attention_row(s[cut:], V[cut:])[:3] if cut < n else ident]
        m, l, a = oracle.attn_merge(parts[0], parts[1])
        assert m == m_all
        assert l == pytest.approx(l_all, rel=1e-14)
        assert np.allclose(a / l, o_all, rtol=1e-13, atol=1e-15)
    # three segments merged in either grouping (associativity)
    segs = [(0, 5), (5, 17), (17, n)]
    p = [oracle.online_attention_row(s[a:b], V[a:b])[:3] for a, b in segs]
    left = oracle.attn_merge(oracle.attn_merge(p[0], p[1]), p[2])
    right = oracle.attn_merge(p[0], oracle.attn_merge(p[1], p[2]))
    assert left[0] == right[0]
    assert np.allclose(left[2] / left[1], right[2] / right[1], rtol=1e-14)
    # the identity leaves a state unchanged
    m, l, a = oracle.attn_merge(ident, p[1])
    assert (m, l) == (p[1][0], p[1][1]) and np.array_equal(a, p[1][2])


def test_attn_decode_nan_propagates():
    q = np.ones((1, 1, 4))
    k = np.ones((1, 1, 3, 4))
    v = np.ones((1, 1, 3, 4))
    k[0, 0, 1, 2] = np.nan
    o, lse, _, _ = oracle.attn_decode(q, k, v)
    assert np.all(np.isnan(o)) and np.isnan(lse[0, 0])


# ------------------------------------------------------------------ softmax backward


def test_softmax_backward_matches_finite_differences():
    """dx is the gradient of L(x) = sum_j dy_j softmax(x)_j: its dot product
    with a direction u equals the central difference of L along u (forward
    oracle, fp64), for several random rows and directions."""
    rng = np.random.default_rng(81)
    for n in (1, 2, 7, 40):
        x = rng.normal(size=n) * 2
        dy = rng.normal(size=n)
        y = oracle.softmax_f64(x)
        dx, _ = oracle.softmax_backward_rows(y[None].astype(np.float32), dy[None].astype(np.float32))
        yf, dyf = y.astype(np.float32).astype(np.float64), dy.astype(np.float32).astype(np.float64)
        dx_exact = yf * (dyf - (dyf * yf).sum())  # same inputs as the oracle saw
        assert np.allclose(dx[0], dx_exact, rtol=1e-14, atol=1e-16)
        for _ in range(3):
            u = rng.normal(size=n)
            eps = 1e-6
            Lp = float(dyf @ oracle.softmax_f64(x + eps * u))
            Lm = float(dyf @ oracle.softmax_f64(x - eps * u))
            # the gradient formula evaluated at the exact y of x
            g = y * (dyf - (dyf * y).sum())
            assert float(g @ u) == pytest.approx((Lp - Lm) / (2 * eps), rel=1e-6, abs=1e-9)


def test_softmax_backward_closed_forms():
    rng = np.random.default_rng(82)
    y = oracle.softmax_f64(rng.normal(size=9)).astype(np.float32)[None]
    yd = y.astype(np.float64)[0]
    # dy constant: dx = y (c - c sum y), zero up to the rounding of sum y
    dx, _ = oracle.softmax_backward_rows(y, np.full_like(y, 3.0))
    assert np.allclose(dx, 3.0 * yd * (1 - yd.sum()), rtol=0, atol=1e-15)
    # dy = e_i: dx_j = y_j (delta_ij - y_i)
    for i in (0, 4, 8):
        e = np.zeros_like(y)
        e[0, i] = 1
        dx, mag = oracle.softmax_backward_rows(y, e)
        want = yd * ((np.arange(9) == i) - yd[i])
        assert np.allclose(dx[0], want, rtol=1e-15, atol=1e-18)
        assert np.all(mag[0] >= np.abs(dx[0]) - 1e-18)


def test_softmax_backward_ragged_rows():
    rng = np.random.default_rng(83)
    y = rng.random((4, 10)).astype(np.float32)
    dy = rng.normal(size=(4, 10)).astype(np.float32)
    L = np.array([0, 3, 10, 12], dtype=np.int32)
    dx, _ = oracle.softmax_backward_rows(y, dy, lengths=L)
    assert np.all(np.isnan(dx[0])) and np.all(np.isnan(dx[1, 3:]))
    full, _ = oracle.softmax_backward_rows(y[1:2, :3].copy(), dy[1:2, :3].copy())
    assert np.array_equal(dx[1, :3], full[0])
    assert not np.isnan(dx[2:]).any()


# ------------------------------------------------------- pointwise ([Stax4] 9.3)


def test_add_2d_transposed_by_hand():
    # Example 6.1 in small: x is 2 x 3, out = x.t() + y is 3 x 2
    x = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float32)
    y = np.array([[10, 20], [30, 40], [50, 60]], dtype=np.float32)
    out = oracle.add_2d(x.T, y)
    assert out.tolist() == [[11, 24], [32, 45], [53, 66]]
    # the other operand transposed, and both
    assert oracle.add_2d(y, x.T).tolist() == [[11, 24], [32, 45], [53, 66]]
    assert oracle.add_2d(x.T, x.T).tolist() == [[2, 8], [4, 10], [6, 12]]


def test_add_2d_rounds_once_to_nearest_even():
    u = 2.0 ** -24  # half an fp32 ulp of 1
    a = np.array([[1.0, 1.0 + 2 * u, 1.0, 1.0]], dtype=np.float32)
    b = np.array([[u, u, 1.5 * u, 0.5 * u]], dtype=np.float32)
    out = oracle.add_2d(a, b)
    # ties go to the even significand; above half rounds up, below down
    assert out.tolist()[0] == [1.0, 1.0 + 4 * u, 1.0 + 2 * u, 1.0]


def test_add_2d_equals_fp32_addition_on_strided_views():
    rng = np.random.default_rng(91)
    x = rng.normal(size=(53, 37)).astype(np.float32) * np.float32(1e3)
    y = rng.normal(size=(37, 60)).astype(np.float32)
    want = x.T + y[:, :53]  # numpy's fp32 add is correctly rounded
    assert np.array_equal(oracle.add_2d(x.T, y[:, :53]), want)
    z = rng.normal(size=(74, 106)).astype(np.float32)
    assert np.array_equal(oracle.add_2d(z[::2, ::2], z[1::2, 1::2]), z[::2, ::2] + z[1::2, 1::2])


def test_gelu_backward_matches_finite_differences():
    # GELU(h) = h Phi(h) with Phi from scipy; dx / dy is its derivative
    gelu = lambda t: t * scipy.special.ndtr(t)  # noqa: E731
    h = np.array([-6.0, -3.0, -1.3, -0.75, -0.2, 0.0, 0.4, 1.0, 2.5, 5.0])
    eps = 1e-6
    fd = (gelu(h + eps) - gelu(h - eps)) / (2 * eps)
    dx, mag = oracle.gelu_backward(1.0, h)
    assert np.allclose(dx, fd, rtol=1e-7, atol=1e-9)
    assert np.all(mag >= np.abs(dx))


def test_gelu_backward_closed_forms():
    dx, _ = oracle.gelu_backward(1.0, np.array([0.0, 1.0, 40.0, -40.0]))
    assert dx[0] == 0.5  # Phi(0) = 1/2
    # Phi(1) + phi(1), textbook values of the normal distribution and density
    assert dx[1] == pytest.approx(0.8413447460685429 + 0.24197072451914337, rel=1e-15)
    assert dx[2] == 1.0 and dx[3] == 0.0
    # GELU'(h) + GELU'(-h) = 1 (Phi(-h) = 1 - Phi(h), phi even)
    h = np.linspace(-5, 5, 41)
    a, _ = oracle.gelu_backward(1.0, h)
    b, _ = oracle.gelu_backward(1.0, -h)
    assert np.allclose(a + b, 1.0, rtol=0, atol=1e-15)
    # GELU has its minimum near h = -0.7518: the derivative changes sign there
    d, _ = oracle.gelu_backward(1.0, np.array([-0.76, -0.74]))
    assert d[0] < 0 < d[1]


def test_gelu_backward_broadcasts_one_upstream_value():
    h = np.linspace(-3, 3, 7)
    one, _ = oracle.gelu_backward(np.array([-2.5]), h)
    each, _ = oracle.gelu_backward(np.full(7, -2.5), h)
    unit, _ = oracle.gelu_backward(1.0, h)
    assert np.array_equal(one, each) and np.array_equal(one, -2.5 * unit)
    g = np.arange(1, 8, dtype=np.float64)
    per, _ = oracle.gelu_backward(g, h)
    assert np.allclose(per, g * unit, rtol=1e-15)


def test_round_bf16_is_the_scalar_rounding_elementwise():
    v = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.0, 0.0, -0.0, math.inf, 3.4e38, 1e-40, -5.5e-3])
    assert oracle.round_bf16(v).tolist() == [oracle.f64_to_bf16(x) for x in v]


# -------------------------------------------------------------- LayerNorm backward


def _ln_forward64(x, gamma, beta, eps):
    """The LayerNorm definition in fp64 numpy (biased variance), for finite
    differences: an independent statement of the forward pass."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def _bf16_rows(rng, shape, scale=1.0, shift=0.0):
    bits = synth.to_bf16((rng.normal(size=shape) * scale + shift).astype(np.float32))
    return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_layernorm_stats_match_numpy():
    rng = np.random.default_rng(101)
    xb, x = _bf16_rows(rng, (5, 300), scale=3.0, shift=7.0)
    mean, rstd = oracle.layernorm_stats(xb, eps=1e-5)
    assert np.allclose(mean, x.mean(axis=1), rtol=1e-14)
    assert np.allclose(rstd, 1.0 / np.sqrt(x.var(axis=1) + 1e-5), rtol=1e-13)


def test_layernorm_backward_matches_finite_differences():
    rng = np.random.default_rng(102)
    rows, cols, eps = 3, 37, 1e-5
    xb, x = _bf16_rows(rng, (rows, cols), scale=2.0, shift=0.5)
    dyb, dy = _bf16_rows(rng, (rows, cols))
    gb, g = _bf16_rows(rng, (cols,), scale=0.5, shift=1.0)
    beta = rng.normal(size=cols)
    mean, rstd = oracle.layernorm_stats(xb, eps)
    out = oracle.layernorm_backward_rows(xb, dyb, gb, mean, rstd)
    L = lambda xx, gg: float((dy * _ln_forward64(xx, gg, beta, eps)).sum())  # noqa: E731
    h = 1e-6
    for _ in range(4):
        u = rng.normal(size=(rows, cols))
        fd = (L(x + h * u, g) - L(x - h * u, g)) / (2 * h)
        assert float((out["dx64"] * u).sum()) == pytest.approx(fd, rel=1e-6, abs=1e-8)
        v = rng.normal(size=cols)
        fd = (L(x, g + h * v) - L(x, g - h * v)) / (2 * h)
        assert float(out["dgamma64"] @ v) == pytest.approx(fd, rel=1e-6, abs=1e-8)
    assert np.allclose(out["dbeta64"], dy.sum(axis=0), rtol=1e-15, atol=0)
    assert np.all(out["dxmag"] >= np.abs(out["dx64"]) - 1e-12)
    assert np.all(out["gmag"] >= np.abs(out["dgamma64"])) and np.all(out["bmag"] >= np.abs(out["dbeta64"]))


def test_layernorm_backward_closed_forms():
    # x-hat = +-1 exactly (mean 2, variance 1, eps 0); dy = x-hat gives dx = 0
    xb = synth.to_bf16(np.array([[1, 3, 1, 3, 3, 1]], dtype=np.float32))
    mean, rstd = oracle.layernorm_stats(xb, eps=0.0)
    assert mean[0] == 2.0 and rstd[0] == 1.0
    dyb = synth.to_bf16(np.array([[-1, 1, -1, 1, 1, -1]], dtype=np.float32))
    out = oracle.layernorm_backward_rows(xb, dyb, None, mean, rstd)
    assert np.all(out["dx64"] == 0.0)
    assert out["dgamma64"].tolist() == [1.0] * 6 and out["dbeta64"].tolist() == [-1, 1, -1, 1, 1, -1]
    # a constant dy (gamma 1) gives dx = 0
    rng = np.random.default_rng(103)
    xb, _ = _bf16_rows(rng, (4, 50))
    mean, rstd = oracle.layernorm_stats(xb, eps=1e-5)
    out = oracle.layernorm_backward_rows(xb, synth.to_bf16(np.full((4, 50), 0.75, np.float32)), None, mean, rstd)
    assert np.allclose(out["dx64"], 0.0, atol=1e-13)


def test_layernorm_backward_invariants():
    # with exact statistics: sum_j dx_j = 0; with eps = 0 also sum_j dx_j xh_j = 0
    rng = np.random.default_rng(104)
    xb, x = _bf16_rows(rng, (6, 129), scale=4.0, shift=-3.0)
    dyb, _ = _bf16_rows(rng, (6, 129))
    gb, _ = _bf16_rows(rng, (129,), scale=0.3, shift=1.0)
    mean, rstd = oracle.layernorm_stats(xb, eps=0.0)
    dx = oracle.layernorm_backward_rows(xb, dyb, gb, mean, rstd)["dx64"]
    xh = (x - mean[:, None]) * rstd[:, None]
    assert np.allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    assert np.allclose((dx * xh).sum(axis=1), 0.0, atol=1e-12)


# ------------------------------------------------------ attention, many query rows


def test_attn_fwd_worked_example(golden):
    """[HG12] 12.1 as a block of one query row: o = [2.6456, 0.9278]."""
    g = golden("hello_gpu_ch12_worked_example.txt")
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[s, 0.0] for s in g["scores"]]]])
    v = np.array([[g["values"]]])
    o, lse, _, _ = oracle.attn_fwd(q, k, v, scale=1.0)
    assert np.allclose(o[0, 0, 0], g["output"], atol=g["tolerance"])
    assert lse[0, 0, 0] == pytest.approx(4 + np.log(g["exp_sum"]), abs=g["tolerance"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(7, 7), (5, 9), (9, 5)])
def test_attn_fwd_matches_a_matrix_statement(causal, nq, nk):
    """softmax(scale Q K^T + mask) V with scipy's softmax and logsumexp and
    numpy's matmul, grouped heads by repetition: an independent statement."""
    rng = np.random.default_rng(nq * 10 + nk + causal)
    B, Hq, Hkv, D = 2, 4, 2, 6
    q = rng.normal(size=(B, Hq, nq, D))
    k = rng.normal(size=(B, Hkv, nk, D))
    v = rng.normal(size=(B, Hkv, nk, D))
    scale = 0.37
    o, lse, mag, smag = oracle.attn_fwd(q, k, v, causal=causal, scale=scale)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    s = scale * (q @ kr.transpose(0, 1, 3, 2))
    if causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    assert np.allclose(o, p @ vr, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-13, atol=1e-13)
    assert np.allclose(mag, p @ np.abs(vr), rtol=1e-12, atol=1e-13)
    assert np.all(mag >= np.abs(o) - 1e-12)


def test_attn_fwd_rows_are_decode_rows():
    # a causal row i is the decode query over the first i + 1 keys
    rng = np.random.default_rng(7)
    q = rng.normal(size=(1, 2, 6, 4))
    k = rng.normal(size=(1, 1, 6, 4))
    v = rng.normal(size=(1, 1, 6, 4))
    o, lse, _, _ = oracle.attn_fwd(q, k, v, causal=True)
    for i in range(6):
        od, ld, _, _ = oracle.attn_decode(q[:, :, i], k, v, lengths=np.array([i + 1], np.int32))
        assert np.allclose(o[:, :, i], od, rtol=1e-14, atol=1e-15) and np.allclose(lse[:, :, i], ld, rtol=1e-14)


def test_attn_fwd_key_permutation_and_shift():
    # without the mask the keys form a set: permuting keys and values together
    # changes nothing; adding scale-invisible u to every key shifts lse only
    rng = np.random.default_rng(8)
    q = rng.normal(size=(1, 1, 5, 3))
    k = rng.normal(size=(1, 1, 8, 3))
    v = rng.normal(size=(1, 1, 8, 3))
    o, lse, _, _ = oracle.attn_fwd(q, k, v)
    perm = rng.permutation(8)
    o2, lse2, _, _ = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm])
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-14)
    u = rng.normal(size=3)
    o3, lse3, _, _ = oracle.attn_fwd(q, k + u, v)
    assert np.allclose(o, o3, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse3, lse + (q[0, 0] @ u) / np.sqrt(3), rtol=1e-12)


def test_row_functions_do_not_depend_on_the_thread_count():
    # the host-thread split only hands out row ranges; every row is the same
    # sequential loop, so one and eight threads give the same bits (the
    # all-cores cpu_baseline times exactly these calls)
    x = synth.normal((37, 515), seed=17) * 3
    L = np.array([(i * 97) % 516 for i in range(37)], np.int32)
    for t in (2, 8):
        y1, a1 = oracle.softmax_rows(x, lengths=L)
        yt, at = oracle.softmax_rows(x, lengths=L, threads=t)
        assert np.array_equal(y1, yt, equal_nan=True) and np.array_equal(a1, at)
        b = synth.uniform((37, 515), seed=18)
        assert all(np.array_equal(u, v) for u, v in zip(oracle.sum_relu_add(x, b), oracle.sum_relu_add(x, b, threads=t)))
        assert np.array_equal(oracle.sumsq_rows(x), oracle.sumsq_rows(x, threads=t))
        xb = synth.to_bf16(x)
        assert all(np.array_equal(u, v) for u, v in zip(oracle.layernorm_rows(xb), oracle.layernorm_rows(xb, threads=t)))
    # the whole-vector sum over slices reorders fp64 additions only: both
    # orders lie within n * 2^-53 (relative) of the exact sum of these
    # nonnegative terms
    v = synth.uniform((100_003,), seed=19)
    exact = math.fsum(float(t) * float(t) for t in v)
    for t in (1, 8):
        assert math.isclose(oracle.sumsq(v, threads=t), exact, rel_tol=v.size * 2.0**-53)
