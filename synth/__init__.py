"""Seeded synthetic inputs shared by the fp64 oracle and the GPU path.

This package draws numbers and does nothing else: it holds none of the
arithmetic of the reductions. Both ``oracle`` and the tests/benchmark of
``pointwise_reduction_amd`` consume what it produces; it imports neither.

The generator is a counter-based SplitMix64 written in C (``synth.c``). Being
counter based, any slice of a stream can be drawn on its own, so large arrays
are drawn in slices on a few threads (ctypes releases the GIL); the values do
not depend on the split. Every function returns numpy arrays.

Workload recipes (the sizes and distributions of the five configurations):

* ``sum_relu_add_inputs``   a, b ~ U(-1, 1) fp32 [rows, cols]; optional NaNs.
* ``softmax_inputs``        x ~ N(0,1)*4 fp32, 1% of entries set to +/-30.
* ``layernorm_inputs``      x ~ N(0.5, sd=2) bf16, gamma ~ U(0.5,1.5), beta ~ U(-0.1,0.1).
* ``sumsq_inputs``          x ~ U(-1, 1) fp32 [n].
* ``ragged_softmax_inputs`` lengths from {1000, 3000, 50257, 131071}, x ~ N(0,1)*3,
                            padded tail filled with NaN.
"""
import concurrent.futures
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SYNTH_LIB names another build (the sanitizer run of the CPU tests)
_SO = os.environ.get("SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
_lib = None

I64, U64, F64, I32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int32
P = ctypes.c_void_p


def build(verbose=False, out=None, cc="gcc", extra=None):
    """Compile synth.c into libsynth.so. `out`, `cc` and `extra` flags serve
    the sanitized build of the CPU tests."""
    flags = ["-O2"] if extra is None else list(extra)
    cmd = [cc] + flags + ["-std=c11", "-shared", "-fPIC", "-o", out or _SO, os.path.join(_HERE, "synth.c"), "-lm"]
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
        "syn_u64": (U64, [U64, U64, U64]),
        "syn_uniform_f32_at": (None, [P, I64, U64, U64, I64, F64, F64]),
        "syn_normal_f32_at": (None, [P, I64, U64, U64, I64, F64, F64]),
        "syn_spiky_normal_rows_range": (None, [P, I64, I64, I64, I64, U64, F64, F64, F64]),
        "syn_lengths": (None, [P, I64, U64, P, I32]),
        "syn_ragged_normal_rows_range": (None, [P, I64, I64, I64, P, U64, F64, F64, ctypes.c_float]),
        "syn_pick_cells": (I32, [I64, I64, U64, U64, I32, P, P]),
        "syn_f32_to_bf16": (None, [P, P, I64]),
        "syn_bf16_to_f32": (None, [P, P, I64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _addr(a, offset_elems=0):
    return ctypes.c_void_p(a.ctypes.data + offset_elems * a.itemsize)


def threads():
    """Threads for large draws: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_SLICE_MIN = 1 << 20  # below this many units one thread does it all


def _parallel(n, fn):
    """Run fn(lo, hi) over [0, n) in contiguous slices, one per thread."""
    t = threads() if n >= _SLICE_MIN else 1
    if t <= 1:
        fn(0, n)
        return
    step = (n + t - 1) // t
    with concurrent.futures.ThreadPoolExecutor(t) as ex:
        list(ex.map(lambda lo: fn(lo, min(n, lo + step)), range(0, n, step)))


def u64(seed, stream, i):
    return int(_load().syn_u64(seed, stream, i))


def uniform(shape, seed, stream=0, lo=-1.0, hi=1.0):
    out = np.empty(shape, dtype=np.float32)
    f = _load().syn_uniform_f32_at
    _parallel(out.size, lambda a, b: f(_addr(out, a), b - a, seed, stream, a, lo, hi))
    return out


def normal(shape, seed, stream=0, mean=0.0, std=1.0):
    out = np.empty(shape, dtype=np.float32)
    f = _load().syn_normal_f32_at
    _parallel(out.size, lambda a, b: f(_addr(out, a), b - a, seed, stream, a, mean, std))
    return out


def to_bf16(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    f = _load().syn_f32_to_bf16
    _parallel(x.size, lambda a, b: f(_addr(x, a), _addr(out, a), b - a))
    return out


def bf16_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    f = _load().syn_bf16_to_f32
    _parallel(b.size, lambda a, c: f(_addr(b, a), _addr(out, a), c - a))
    return out


def _parallel_rows(rows, row_elems, fn):
    """Run fn(r0, r1) over row ranges; slices hold whole rows."""
    if rows * row_elems < _SLICE_MIN or rows < 2:
        fn(0, rows)
        return
    t = min(threads(), rows)
    step = (rows + t - 1) // t
    with concurrent.futures.ThreadPoolExecutor(t) as ex:
        list(ex.map(lambda r0: fn(r0, min(rows, r0 + step)), range(0, rows, step)))


def pick_cells(rows, cols, seed, stream, count):
    r = np.zeros(count, dtype=np.int32)
    c = np.zeros(count, dtype=np.int32)
    n = _load().syn_pick_cells(rows, cols, seed, stream, count, _p(r), _p(c))
    return r[:n], c[:n]


# ---------------------------------------------------------------- workloads


def sum_relu_add_inputs(rows=64, cols=128, seed=1001, n_nan=0):
    """a, b ~ U(-1,1) fp32 [rows, cols]. With n_nan > 0, that many NaNs are
    placed at seeded cells in distinct rows, half in a and half in b."""
    a = uniform((rows, cols), seed, stream=0)
    b = uniform((rows, cols), seed, stream=1)
    nan_rows = np.zeros(0, dtype=np.int32)
    if n_nan:
        r, c = pick_cells(rows, cols, seed, 0, n_nan)
        half = (len(r) + 1) // 2
        a[r[:half], c[:half]] = np.nan
        b[r[half:], c[half:]] = np.nan
        nan_rows = np.sort(r)
    return a, b, nan_rows


def softmax_inputs(rows=4096, cols=1024, seed=2001, scale=4.0, p_spike=0.01, spike=30.0, row_stride=None):
    rs = cols if row_stride is None else row_stride
    x = np.zeros((rows, rs), dtype=np.float32)
    f = _load().syn_spiky_normal_rows_range
    _parallel_rows(rows, cols, lambda r0, r1: f(_p(x), r0, r1, cols, rs, seed, scale, p_spike, spike))
    return x


def layernorm_inputs(rows=2048, cols=32768, seed=3001):
    """x ~ N(0.5, sd 2), gamma ~ U(0.5, 1.5), beta ~ U(-0.1, 0.1); all bf16 (uint16 bits)."""
    x = to_bf16(normal((rows, cols), seed, stream=0, mean=0.5, std=2.0))
    g = to_bf16(uniform((cols,), seed, stream=1, lo=0.5, hi=1.5))
    b = to_bf16(uniform((cols,), seed, stream=2, lo=-0.1, hi=0.1))
    return x, g, b


def sumsq_inputs(n=1 << 28, seed=4001):
    return uniform((n,), seed, stream=0)


RAGGED_CHOICES = (1000, 3000, 50257, 131071)


def ragged_lengths(rows=512, seed=5001, choices=RAGGED_CHOICES):
    ch = np.asarray(choices, dtype=np.int32)
    out = np.zeros(rows, dtype=np.int32)
    _load().syn_lengths(_p(out), rows, seed, _p(ch), len(ch))
    return out


def ragged_softmax_inputs(rows=512, row_stride=131072, seed=5001, choices=RAGGED_CHOICES, std=3.0,
                          tail=float("nan"), lengths=None):
    """x ~ N(0,1)*std over each row's valid prefix; the padded tail holds `tail`."""
    L = ragged_lengths(rows, seed, choices) if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    x = np.empty((rows, row_stride), dtype=np.float32)
    f = _load().syn_ragged_normal_rows_range
    _parallel_rows(rows, row_stride, lambda r0, r1: f(_p(x), r0, r1, row_stride, _p(L), seed, 0.0, std, tail))
    return x, L


def attn_decode_inputs(batch=8, heads_q=32, heads_kv=8, seq=8192, dim=128, seed=6001, lengths=None, choices=None,
                       bf16=True, tail=float("nan")):
    """Decode attention: q [B, Hq, D], k, v [B, Hkv, S, D], all N(0, 1); with
    bf16 the values are rounded to bf16 and returned as uint16 bits, else as
    fp32. lengths: explicit [B] valid key counts, or drawn from `choices`,
    or None (every batch has S keys). Keys and values at j >= len_b hold
    `tail` (NaN by default: they must never be read)."""
    q = normal((batch, heads_q, dim), seed, stream=0)
    k = normal((batch, heads_kv, seq, dim), seed, stream=1)
    v = normal((batch, heads_kv, seq, dim), seed, stream=2)
    if lengths is None and choices is not None:
        lengths = ragged_lengths(batch, seed, choices)
    L = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    if L is not None:
        for b in range(batch):
            n = int(np.clip(L[b], 0, seq))
            k[b, :, n:] = tail
            v[b, :, n:] = tail
    if bf16:
        return to_bf16(q), to_bf16(k), to_bf16(v), L
    return q, k, v, L


def attn_block_inputs(batch=4, heads_q=16, heads_kv=16, seq_q=4096, seq_kv=4096, dim=128, seed=7001):
    """Attention over blocks of query rows: q [B, Hq, Nq, D], k, v [B, Hkv, Nk,
    D], all N(0, 1), rounded to bf16 and returned as uint16 bits."""
    q = normal((batch, heads_q, seq_q, dim), seed, stream=0)
    k = normal((batch, heads_kv, seq_kv, dim), seed, stream=1)
    v = normal((batch, heads_kv, seq_kv, dim), seed, stream=2)
    return to_bf16(q), to_bf16(k), to_bf16(v)
