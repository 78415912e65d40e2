"""Helpers shared by the GPU parity tests: device copies, forced forms and
the comparison rules (the tolerances are stated here once)."""
import contextlib
import math

import numpy as np

try:
    import torch
except ImportError:  # CPU-only environments never call these helpers
    torch = None

DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@contextlib.contextmanager
def forced(form):
    import pointwise_reduction_amd as fr
    prev = fr.fr_force_form(form)
    try:
        yield
    finally:
        fr.fr_force_form(prev)


def bf16_bits_tensor(bits_u16):
    """uint16 bit patterns (numpy) -> torch bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_bits_of(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ comparison rules


def check_fp32(got, ref64, terms=None, what=""):
    """fp32 results: |got - ref| <= 1e-5 * sum|terms| + 1e-6 element by element,
    NaN exactly where the reference is NaN, infinities equal. `terms` defaults
    to |ref| (sums of nonnegative terms, and normalized softmax terms, whose
    own magnitude is the bound). Large arrays are checked in slices; elements
    inside the bound pass at once and the rest are examined."""
    got = np.asarray(got)
    ref64 = np.asarray(ref64, dtype=np.float64)
    assert got.shape == ref64.shape, what
    g_all, r_all = got.reshape(-1), ref64.reshape(-1)
    t_all = None if terms is None else np.broadcast_to(np.asarray(terms, dtype=np.float64), ref64.shape).reshape(-1)
    step = 1 << 22
    for lo in range(0, r_all.size, step):
        g = g_all[lo:lo + step].astype(np.float64)
        r = r_all[lo:lo + step]
        t = np.abs(r) if t_all is None else t_all[lo:lo + step]
        with np.errstate(invalid="ignore"):
            ok = (np.abs(g - r) <= 1e-5 * t + 1e-6) & np.isfinite(r)
        if ok.all():
            continue
        rest = np.nonzero(~ok)[0]
        g, r, t = g[rest], r[rest], t[rest]
        nr, ng = np.isnan(r), np.isnan(g)
        if not np.array_equal(nr, ng):
            at = np.unravel_index(int(lo + rest[np.nonzero(nr != ng)[0][0]]), ref64.shape)
            raise AssertionError(f"{what}: NaN mismatch at {tuple(int(i) for i in at)}")
        inf = ~nr & np.isinf(r)
        assert np.array_equal(g[inf], r[inf]), what
        bad = ~nr & ~inf
        with np.errstate(invalid="ignore"):
            bad &= ~(np.abs(g - r) <= 1e-5 * t + 1e-6)
        if bad.any():
            err, bound = np.abs(g - r)[bad], (1e-5 * t + 1e-6)[bad]
            i = int(np.argmax(err - bound))
            raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance in slice at {lo}; worst err "
                                 f"{err[i]:.3e} vs bound {bound[i]:.3e} (ref {r[bad][i]:.9g}, got {g[bad][i]:.9g})")


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def bf16_ulp_of_bits(bits):
    """The ulp of a finite bf16 value from its bit pattern: 2^(e - 134) for a
    biased exponent e >= 1, and 2^-133 for zero and subnormals (the same
    values bf16_ulp gives)."""
    e = ((np.asarray(bits, dtype=np.uint16) >> 7) & 0xFF).astype(np.int32)
    return np.ldexp(1.0, np.maximum(e, 1) - 134)


def check_bf16(got_bits, ref_bits, y64, mag, what=""):
    """bf16 results: within one bf16 ulp of the oracle's bf16 value; or, where
    the result is a near-cancellation (tiny |y| against large terms), within
    the fp32 rule on the terms that form it: 1e-5 * mag + 1e-6. Identical bit
    patterns pass at once; the rule is evaluated on the rest."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16)
    assert got_bits.shape == ref_bits.shape, what
    y64 = np.broadcast_to(np.asarray(y64, dtype=np.float64), ref_bits.shape)
    mag = np.broadcast_to(np.asarray(mag, dtype=np.float64), ref_bits.shape)
    diff = np.nonzero((got_bits != ref_bits).ravel())[0]
    if diff.size == 0:
        return
    gb, rb = got_bits.ravel()[diff], ref_bits.ravel()[diff]
    g, r = bf16_to_f64(gb), bf16_to_f64(rb)
    nr, ng = np.isnan(r), np.isnan(g)
    assert np.array_equal(nr, ng), f"{what}: NaN mismatch"
    fin = ~nr
    yv, mv = y64.ravel()[diff], mag.ravel()[diff]
    with np.errstate(invalid="ignore"):
        ok = np.abs(g - r) <= bf16_ulp_of_bits(rb)
        ok |= np.abs(g - yv) <= 1e-5 * mv + 1e-6
    bad = fin & ~ok
    if bad.any():
        idx = [np.unravel_index(int(i), ref_bits.shape) for i in diff[bad][:5]]
        raise AssertionError(f"{what}: {int(bad.sum())} bf16 outputs off by more than one ulp, e.g. at "
                             f"{[tuple(int(t) for t in i) for i in idx]}: got {g[bad][:3]}, ref {r[bad][:3]}, "
                             f"exact {yv[bad][:3]}")


def isclose_sum(got, ref, n_terms_abs):
    return abs(got - ref) <= 1e-5 * n_terms_abs + 1e-6 or (math.isnan(got) and math.isnan(ref))
