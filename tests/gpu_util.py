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
    NaN exactly where the reference is NaN. `terms` defaults to |ref| (sums of
    nonnegative terms, and normalized softmax terms, whose own magnitude is the
    bound)."""
    got = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    assert got.shape == ref64.shape, what
    nr, ng = np.isnan(ref64), np.isnan(got)
    assert np.array_equal(nr, ng), f"{what}: NaN mismatch at {np.argwhere(nr != ng)[:5].tolist()}"
    fin = ~nr
    bound = 1e-5 * (np.abs(ref64) if terms is None else np.asarray(terms, dtype=np.float64)) + 1e-6
    inf = fin & np.isinf(ref64)
    assert np.array_equal(got[inf], ref64[inf]), what
    fin &= ~inf
    err = np.abs(got[fin] - ref64[fin])
    bad = err > bound[fin]
    if bad.any():
        i = np.argmax(err - bound[fin])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst err {err[i]:.3e} "
                             f"vs bound {bound[fin][i]:.3e} (ref {ref64[fin][i]:.9g}, got {got[fin][i]:.9g})")


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def check_bf16(got_bits, ref_bits, y64, mag, what=""):
    """bf16 results: within one bf16 ulp of the oracle's bf16 value; or, where
    the result is a near-cancellation (tiny |y| against large terms), within
    the fp32 rule on the terms that form it: 1e-5 * mag + 1e-6."""
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    nr, ng = np.isnan(r), np.isnan(g)
    assert np.array_equal(nr, ng), f"{what}: NaN mismatch"
    fin = ~nr
    ok = np.abs(g - r) <= bf16_ulp(r)
    ok |= np.abs(g - y64) <= 1e-5 * mag + 1e-6
    bad = fin & ~ok
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} bf16 outputs off by more than one ulp, e.g. at {idx}: "
                             f"got {g[bad][:3]}, ref {r[bad][:3]}, exact {y64[bad][:3]}")


def isclose_sum(got, ref, n_terms_abs):
    return abs(got - ref) <= 1e-5 * n_terms_abs + 1e-6 or (math.isnan(got) and math.isnan(ref))
