"""CPU: the comparison rules every GPU parity test applies (tests/gpu_util.py).

fp32: |got - ref| <= 1e-5 * sum|terms| + 1e-6 per element, NaN exactly where
the reference is NaN, infinities equal. bf16: within one bf16 ulp of the
oracle's bf16 value, or within the fp32 rule on the terms of a
near-cancellation. These run on planted values: each rule must pass what it
allows and fail what it does not.
"""
import numpy as np
import pytest

from gpu_util import bf16_to_f64, bf16_ulp, bf16_ulp_of_bits, check_bf16, check_fp32


def test_fp32_rule():
    ref = np.array([np.nan, 1.0, np.inf, -np.inf, 0.5, 0.0, 1e6])
    ok = np.array([np.nan, 1.0 + 9e-6, np.inf, -np.inf, 0.5 + 5.9e-6, 9e-7, 1e6 + 10.0], dtype=np.float64)
    check_fp32(ok, ref)
    for i, bad in [(0, 1.0), (1, np.nan), (2, -np.inf), (3, np.inf), (2, 1e30), (4, 0.5 + 7e-6), (5, 1.2e-6),
                   (6, 1e6 + 10.5)]:
        g = ok.copy()
        g[i] = bad
        with pytest.raises(AssertionError):
            check_fp32(g, ref)


def test_fp32_rule_with_terms_and_large_arrays():
    ref = np.zeros(5_000_000)
    terms = np.full(ref.shape, 100.0)
    got = np.full(ref.shape, 1.0e-3)  # within 1e-5 * 100 + 1e-6
    check_fp32(got, ref, terms=terms)
    got[4_999_999] = 1.1e-3
    with pytest.raises(AssertionError):
        check_fp32(got, ref, terms=terms)


def test_bf16_ulp_from_bits_equals_the_value_rule():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = bf16_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(bf16_ulp(v)[fin], bf16_ulp_of_bits(bits)[fin])
    assert bf16_ulp_of_bits(np.uint16(0x3F80)) == 2.0 ** -7  # 1.0
    assert bf16_ulp_of_bits(np.uint16(0x0001)) == 2.0 ** -133  # smallest subnormal


def test_bf16_rule():
    ref = np.array([0x3F80, 0xBF80, 0x0000, 0x7FC0, 0x4000], dtype=np.uint16)  # 1, -1, 0, NaN, 2
    y64 = bf16_to_f64(ref)
    mag = np.abs(y64)
    got = ref.copy()
    got[0] += 1  # one ulp above 1
    got[1] += 1  # one ulp further from zero
    check_bf16(got, ref, y64, mag)
    for i, delta in [(0, 2), (4, 3)]:
        g = ref.copy()
        g[i] += delta
        with pytest.raises(AssertionError):
            check_bf16(g, ref, y64, mag)
    g = ref.copy()
    g[3] = 0x3F80  # a number where the oracle has NaN
    with pytest.raises(AssertionError):
        check_bf16(g, ref, y64, mag)
    # near-cancellation: tiny exact value against large terms passes on the fp32 rule
    ref2 = np.array([0x2F80], dtype=np.uint16)  # 2^-32
    got2 = np.array([0x3700], dtype=np.uint16)  # 2^-17: far beyond one ulp
    check_bf16(got2, ref2, np.array([2.0 ** -32]), np.array([10.0]))
    with pytest.raises(AssertionError):
        check_bf16(got2, ref2, np.array([2.0 ** -32]), np.array([1e-3]))
