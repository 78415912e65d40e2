"""fp64 CPU oracle for the fused pointwise + row-reduction operations.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``pointwise_reduction_amd``) never imports, loads or calls it, and the two
share no code: the only common dependency is the seeded input generator
(``synth``).

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential loops; each
function cites the passage it implements). This module only compiles it with
gcc and marshals numpy arrays through ctypes. Row-wise functions take a
``threads`` argument: rows are independent, so a large call hands contiguous
row ranges to that many threads, each running the same C loop over its
rows (ctypes releases the GIL). Every row's arithmetic is unchanged, so the
results do not depend on the thread count.
"""
import concurrent.futures
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names another build (the sanitizer run of the CPU tests)
_SO = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

I64, I32, F64, U16 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_uint16
P = ctypes.c_void_p


SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(verbose=False, out=None, cc="gcc", extra=None):
    """Compile oracle.c into liboracle.so (no GPU toolchain involved). `out`,
    `cc` and `extra` flags serve the sanitized build (clang, SANITIZE_FLAGS)."""
    flags = ["-O2"] if extra is None else list(extra)
    cmd = [cc] + flags + ["-std=c11", "-fno-fast-math", "-shared", "-fPIC", "-o", out or _SO,
                          os.path.join(_HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    sig = {
        "orc_bf16_to_double": (F64, [U16]),
        "orc_double_to_bf16": (U16, [F64]),
        "orc_sum_relu_add": (None, [P, P, I64, I64, I64, I64, P, P]),
        "orc_softmax_f64": (None, [P, I64, P]),
        "orc_softmax_rows": (None, [P, I64, I64, I64, P, P, P, I64, P, P]),
        "orc_md_combine": (None, [F64, F64, F64, F64, P, P]),
        "orc_md_fold": (None, [P, I64, P, P]),
        "orc_online_attention_row": (None, [P, P, I64, I64, P, P, P, P]),
        "orc_layernorm_rows": (None, [P, P, P, I64, I64, I64, F64, P, P, P, I64]),
        "orc_sumsq": (F64, [P, I64]),
        "orc_sumsq_rows": (None, [P, I64, I64, I64, P]),
        "orc_softmax_backward_rows": (None, [P, P, I64, I64, I64, I64, P, P, P]),
        "orc_attn_decode": (None, [P, P, P, I64, I64, I64, I64, I64, P, F64, P, P, P, P, P]),
        "orc_attn_merge": (None, [F64, F64, P, F64, F64, P, I64, P, P, P]),
        "orc_add_2d": (None, [P, I64, I64, P, I64, I64, P, I64, I64, I64]),
        "orc_attn_fwd": (None, [P, P, P, I64, I64, I64, I64, I64, I64, I32, F64, P, P, P, P, P]),
        "orc_round_bf16": (None, [P, I64, P]),
        "orc_layernorm_stats": (None, [P, I64, I64, I64, F64, P, P]),
        "orc_layernorm_backward_rows": (None, [P, P, P, P, P, I64, I64, I64, I64, P, P, P, P, P, P]),
        "orc_gelu_backward": (None, [P, I64, P, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def host_threads():
    """The CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _row_ranges(rows, cols, threads):
    """Contiguous row ranges, one per thread; one range for small calls."""
    if threads is None:
        threads = min(16, host_threads()) if rows * max(cols, 1) >= (1 << 20) else 1
    t = max(1, min(int(threads), rows))
    step = (rows + t - 1) // t if rows else 1
    return [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)] or [(0, 0)]


def _run_ranges(ranges, fn):
    if len(ranges) == 1:
        fn(*ranges[0])
        return
    with concurrent.futures.ThreadPoolExecutor(len(ranges)) as ex:
        list(ex.map(lambda rr: fn(*rr), ranges))


def _rows2d(x, dtype):
    """Return (array, rows, cols, row_stride) for a 2-D array whose inner stride is 1."""
    x = np.asarray(x)
    assert x.dtype == dtype and x.ndim == 2
    assert x.strides[1] == x.itemsize, "inner stride must be 1"
    return x, x.shape[0], x.shape[1], x.strides[0] // x.itemsize


# ------------------------------------------------------------------ bf16


def bf16_to_f64(bits):
    return float(_load().orc_bf16_to_double(int(bits)))


def f64_to_bf16(v):
    return int(_load().orc_double_to_bf16(float(v)))


def round_bf16(v):
    """fp64 array -> bf16 bit patterns (uint16), each rounded once to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_round_bf16(_p(v), v.size, _p(out))
    return out


# ------------------------------------------------------------------ C1


def sum_relu_add(a, b, threads=None):
    """out[i] = sum_r 2*relu(a[i,r]+b[i,r]); returns (out fp32, out fp64)."""
    a, rows, cols, a_rs = _rows2d(a, np.float32)
    b, rows_b, cols_b, b_rs = _rows2d(b, np.float32)
    assert (rows, cols) == (rows_b, cols_b)
    out = np.empty(rows, dtype=np.float32)
    out64 = np.empty(rows, dtype=np.float64)
    f = _load().orc_sum_relu_add
    _run_ranges(_row_ranges(rows, cols, threads),
                lambda r0, r1: f(_p(a[r0:r1]), _p(b[r0:r1]), r1 - r0, cols, a_rs, b_rs, _p(out[r0:r1]),
                                 _p(out64[r0:r1])))
    return out, out64


# ------------------------------------------------------------------ softmax


def softmax_f64(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().orc_softmax_f64(_p(x), x.size, _p(y))
    return y


def softmax_rows(x, lengths=None, cols=None, threads=None):
    """Row softmax of fp32 rows (ragged when `lengths` is given).

    x may be a 2-D view with unit inner stride. `cols` (default x.shape[1]) is
    the row capacity lengths are clamped to. Returns (y64, argmax): y64 is a
    float64 array shaped like x[:, :cols] holding NaN wherever the oracle did
    not write (j >= len), argmax is int32 (-1 for an empty row).
    """
    x, rows, xc, x_rs = _rows2d(x, np.float32)
    cols = xc if cols is None else cols
    assert cols <= xc
    L = None
    if lengths is not None:
        L = np.ascontiguousarray(lengths, dtype=np.int32)
        assert L.shape == (rows,)
    y64 = np.full((rows, cols), np.nan, dtype=np.float64)
    am = np.empty(rows, dtype=np.int32)
    f = _load().orc_softmax_rows

    def run(r0, r1):
        scratch = np.empty(2 * max(cols, 1), dtype=np.float64)
        f(_p(x[r0:r1]), r1 - r0, cols, x_rs, None if L is None else _p(L[r0:r1]), None, _p(y64[r0:r1]), cols,
          _p(am[r0:r1]), _p(scratch))

    _run_ranges(_row_ranges(rows, cols, threads), run)
    return y64, am


def softmax_backward_rows(y, dy, lengths=None):
    """dx = y * (dy - sum(dy * y)) per row in fp64 (see orc_softmax_backward_rows).
    y, dy: fp32 [rows, cols] (2-D views with unit inner stride). Returns
    (dx64, mag), NaN past each row's length."""
    y, rows, cols, y_rs = _rows2d(y, np.float32)
    dy, rows2, cols2, dy_rs = _rows2d(dy, np.float32)
    assert (rows2, cols2) == (rows, cols)
    L = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    dx = np.full((rows, cols), np.nan)
    mag = np.full((rows, cols), np.nan)
    _load().orc_softmax_backward_rows(_p(y), _p(dy), rows, cols, y_rs, dy_rs, _p(L), _p(dx), _p(mag))
    return dx, mag


def md_combine(m1, d1, m2, d2):
    m = ctypes.c_double()
    d = ctypes.c_double()
    _load().orc_md_combine(m1, d1, m2, d2, ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def md_fold(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    m = ctypes.c_double()
    d = ctypes.c_double()
    _load().orc_md_fold(_p(x), x.size, ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def online_attention_row(scores, V):
    """(m, l, a, o) after the online update over all scores ([HG12] 12.3)."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, dv = V.shape
    assert s.shape == (n,)
    a = np.empty(dv)
    o = np.empty(dv)
    m = ctypes.c_double()
    l = ctypes.c_double()
    _load().orc_online_attention_row(_p(s), _p(V), n, dv, ctypes.byref(m), ctypes.byref(l), _p(a), _p(o))
    return m.value, l.value, a, o


# ------------------------------------------------------------------ attention decode


def attn_decode(q, k, v, lengths=None, scale=None):
    """Decode attention ([Stax4] 9.10; [HG12] 12.1) in fp64.

    q: [B, Hq, D]; k, v: [B, Hkv, S, D] (any float dtype; bf16 callers pass
    decoded values). Returns (o64 [B, Hq, D], lse [B, Hq], mag [B, Hq, D],
    smag [B, Hq]) as defined at orc_attn_decode."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    assert (Bk, Dk) == (B, D) and v.shape == k.shape and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    L = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    assert L is None or L.shape == (B,)
    o = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    mag = np.empty((B, Hq, D))
    smag = np.empty((B, Hq))
    scratch = np.empty(max(S, 1))
    _load().orc_attn_decode(_p(q), _p(k), _p(v), B, Hq, Hkv, S, D, _p(L), float(scale), _p(scratch), _p(o), _p(lse),
                            _p(mag), _p(smag))
    return o, lse, mag, smag


def attn_fwd(q, k, v, causal=False, scale=None):
    """Attention of blocks of query rows ([Stax4] 9.10) in fp64.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D] (any float dtype; bf16 callers
    pass decoded values). Returns (o64 [B, Hq, Nq, D], lse [B, Hq, Nq],
    mag [B, Hq, Nq, D], smag [B, Hq, Nq]) as defined at orc_attn_fwd."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    assert (Bk, Dk) == (B, D) and v.shape == k.shape and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty((B, Hq, Nq, D))
    lse = np.empty((B, Hq, Nq))
    mag = np.empty((B, Hq, Nq, D))
    smag = np.empty((B, Hq, Nq))
    scratch = np.empty(max(Nk, 1))
    _load().orc_attn_fwd(_p(q), _p(k), _p(v), B, Hq, Hkv, Nq, Nk, D, int(bool(causal)), float(scale), _p(scratch),
                         _p(o), _p(lse), _p(mag), _p(smag))
    return o, lse, mag, smag


def attn_merge(p1, p2):
    """(m, l, a) (+) (m, l, a) ([Stax4] 9.10)."""
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    a1 = np.ascontiguousarray(a1, dtype=np.float64)
    a2 = np.ascontiguousarray(a2, dtype=np.float64)
    a = np.empty_like(a1)
    m = ctypes.c_double()
    l = ctypes.c_double()
    _load().orc_attn_merge(float(m1), float(l1), _p(a1), float(m2), float(l2), _p(a2), a1.shape[0], ctypes.byref(m),
                           ctypes.byref(l), _p(a))
    return m.value, l.value, a


# ------------------------------------------------------------------ LayerNorm


def layernorm_rows(x_bf16, gamma=None, beta=None, eps=1e-5, threads=None):
    """LayerNorm over rows of bf16 bits (uint16). Returns (y_bf16, y64, mag)."""
    x, rows, cols, x_rs = _rows2d(x_bf16, np.uint16)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.uint16)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.uint16)
    y = np.empty((rows, cols), dtype=np.uint16)
    y64 = np.empty((rows, cols), dtype=np.float64)
    mag = np.empty((rows, cols), dtype=np.float64)
    f = _load().orc_layernorm_rows
    _run_ranges(_row_ranges(rows, cols, threads),
                lambda r0, r1: f(_p(x[r0:r1]), _p(g), _p(b), r1 - r0, cols, x_rs, float(eps), _p(y[r0:r1]),
                                 _p(y64[r0:r1]), _p(mag[r0:r1]), cols))
    return y, y64, mag


def layernorm_stats(x_bf16, eps=1e-5):
    """(mean, rstd) per row in fp64, as the forward pass saves them."""
    x, rows, cols, x_rs = _rows2d(x_bf16, np.uint16)
    mean = np.empty(rows)
    rstd = np.empty(rows)
    _load().orc_layernorm_stats(_p(x), rows, cols, x_rs, float(eps), _p(mean), _p(rstd))
    return mean, rstd


def layernorm_backward_rows(x_bf16, dy_bf16, gamma, mean, rstd):
    """LayerNorm backward from saved (mean, rstd) (see orc_layernorm_backward_rows).
    x, dy: bf16 bits [rows, cols]; gamma: bf16 bits [cols] or None; mean, rstd:
    [rows] values (any float dtype). Returns a dict with dx64, dxmag [rows, cols]
    and dgamma64, dbeta64, gmag, bmag [cols]."""
    x, rows, cols, x_rs = _rows2d(x_bf16, np.uint16)
    dy, r2, c2, dy_rs = _rows2d(dy_bf16, np.uint16)
    assert (r2, c2) == (rows, cols)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.uint16)
    mean = np.ascontiguousarray(mean, dtype=np.float64)
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    assert mean.size == rows and rstd.size == rows
    out = {k: np.empty((rows, cols)) for k in ("dx64", "dxmag")}
    out.update({k: np.empty(cols) for k in ("dgamma64", "dbeta64", "gmag", "bmag")})
    _load().orc_layernorm_backward_rows(_p(x), _p(dy), _p(g), _p(mean), _p(rstd), rows, cols, x_rs, dy_rs,
                                        *(_p(out[k]) for k in ("dx64", "dxmag", "dgamma64", "dbeta64", "gmag",
                                                               "bmag")))
    return out


# ------------------------------------------------------------------ sum of squares


def sumsq(x, threads=1):
    """sum of x^2 in fp64. threads > 1 (the all-cores timing leg only) sums
    equal contiguous slices on separate threads and adds the slice sums in
    slice order: the same terms in another fp64 order, a difference far
    below any tolerance. Parity checks use the sequential sum (threads=1)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    f = _load().orc_sumsq
    t = max(1, min(int(threads), x.size))
    if t == 1:
        return float(f(_p(x), x.size))
    step = (x.size + t - 1) // t
    parts = [None] * t
    def run(i):
        seg = x[i * step:(i + 1) * step]
        parts[i] = float(f(_p(seg), seg.size))
    with concurrent.futures.ThreadPoolExecutor(t) as ex:
        list(ex.map(run, range(t)))
    total = 0.0
    for v in parts:
        total += v
    return total


def sumsq_rows(x, threads=None):
    x, rows, cols, rs = _rows2d(x, np.float32)
    out = np.empty(rows, dtype=np.float64)
    f = _load().orc_sumsq_rows
    _run_ranges(_row_ranges(rows, cols, threads), lambda r0, r1: f(_p(x[r0:r1]), r1 - r0, cols, rs, _p(out[r0:r1])))
    return out


# ------------------------------------------------------------------ pointwise


def _elem_strides(x):
    assert all(st % x.itemsize == 0 and st >= 0 for st in x.strides)
    return [st // x.itemsize for st in x.strides]


def add_2d(a, b):
    """out = a + b for fp32 2-D arrays of one shape; either may be a strided
    view (a transposed array, [Stax4] 9.3 Example 6.1). Returns a contiguous
    fp32 array, each element the correctly rounded fp32 sum."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.dtype == np.float32 and b.dtype == np.float32 and a.ndim == 2 and a.shape == b.shape
    rows, cols = a.shape
    (a_rs, a_cs), (b_rs, b_cs) = _elem_strides(a), _elem_strides(b)
    out = np.empty((rows, cols), dtype=np.float32)
    _load().orc_add_2d(_p(a), a_rs, a_cs, _p(b), b_rs, b_cs, _p(out), cols, rows, cols)
    return out


def gelu_backward(dy, h):
    """dx = dy * (Phi(h) + h phi(h)) in fp64 ([Stax4] 9.3, Listing 9.3).
    h: 1-D values (any float dtype; bf16 callers convert first). dy: one
    value (broadcast) or an array shaped like h. Returns (dx64, mag)."""
    h = np.ascontiguousarray(h, dtype=np.float64).ravel()
    dy = np.ascontiguousarray(dy, dtype=np.float64).ravel()
    assert dy.size in (1, h.size)
    stride = 0 if dy.size == 1 and h.size != 1 else 1
    dx = np.empty(h.size)
    mag = np.empty(h.size)
    _load().orc_gelu_backward(_p(dy), stride, _p(h), h.size, _p(dx), _p(mag))
    return dx, mag
