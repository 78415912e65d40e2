"""GPU parity: fr_attn_decode against the fp64 oracle.

Decode attention ("Stax (4)", 9.10; hello-gpu, Chapter 12, 12.1): one query
row per (batch, query head), grouped query heads, optional per-batch key
lengths (the key/value tail beyond a length holds NaN and must never be
read), fp32 and bf16 data with fp32 arithmetic.
Tolerances: fp32 o within 1e-5 * sum_j p_j |v_jd| + 1e-6 of the exact value;
bf16 o within one bf16 ulp of the oracle's rounded value (or the fp32 rule
for near-cancellations); lse within 1e-5 * (1 + max_j sum_d |scale q_d k_jd|).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_of, bf16_bits_tensor, bf16_to_f64, check_bf16, check_fp32, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


def to_dev(a, bf16):
    return bf16_bits_tensor(a) if bf16 else dev(a)


def run(q, k, v, lengths=None, scale=None, bf16=True, want_lse=True):
    qd, kd, vd = (to_dev(t, bf16) for t in (q, k, v))
    o = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device="cuda")
    lse = torch.full(qd.shape[:2], 7.0, dtype=torch.float32, device="cuda") if want_lse else None
    L = None if lengths is None else dev(np.asarray(lengths, dtype=np.int32))
    fr.fr_attn_decode(qd, kd, vd, o, lse=lse, lengths=L, scale=scale)
    got = bf16_bits_of(o) if bf16 else host(o)
    return got, (host(lse) if want_lse else None)


def reference(q, k, v, lengths, scale, bf16):
    f = bf16_to_f64 if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    return oracle.attn_decode(f(q), f(k), f(v), lengths=lengths, scale=scale)


def compare(q, k, v, got, lse, lengths=None, scale=None, bf16=True, what=""):
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o64, lse64, mag, smag = reference(q, k, v, lengths, scale, bf16)
    if bf16:
        ref_bits = np.vectorize(oracle.f64_to_bf16, otypes=[np.uint16])(o64)
        check_bf16(got, ref_bits, o64, mag, what=what)
    else:
        check_fp32(got, o64, terms=mag, what=what)
    if lse is not None:
        fin = np.isfinite(lse64)
        assert np.array_equal(np.isneginf(lse), np.isneginf(lse64)), what
        err = np.abs(lse[fin] - lse64[fin])
        assert np.all(err <= 1e-5 * (1 + smag[fin])), f"{what}: lse off by {err.max():.3e}"


def test_attn_decode_worked_example(golden):
    """[HG12] 12.1 on the device: scores [2, 1, 4] and values [1,0], [0,2],
    [3,1], embedded in dim 64 (the other coordinates 0), scale 1."""
    g = golden("hello_gpu_ch12_worked_example.txt")
    D = 64
    q = np.zeros((1, 1, D), dtype=np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 3, D), dtype=np.float32)
    k[0, 0, :, 0] = g["scores"]
    v = np.zeros((1, 1, 3, D), dtype=np.float32)
    v[0, 0, :, :2] = g["values"]
    got, lse = run(q, k, v, scale=1.0, bf16=False)
    assert np.allclose(got[0, 0, :2], g["output"], atol=g["tolerance"])
    assert np.all(got[0, 0, 2:] == 0)
    assert lse[0, 0] == pytest.approx(np.log(np.exp(2) + np.exp(1) + np.exp(4)), rel=1e-6)
    compare(q, k, v, got, lse, scale=1.0, bf16=False, what="worked example")


CASES = [
    # (B, Hq, Hkv, S, D, bf16, length choices)
    (2, 8, 8, 1000, 128, True, None),
    (2, 8, 2, 777, 128, True, (0, 1, 255, 256, 257, 777)),
    (3, 16, 2, 513, 128, False, (1, 300, 513)),
    (2, 8, 1, 300, 128, True, None),
    (4, 4, 4, 600, 64, True, (2, 600)),
    (2, 16, 4, 1100, 64, False, None),
    (1, 2, 1, 256, 64, True, None),
    (1, 1, 1, 1, 128, False, None),
    (2, 4, 2, 20000, 64, True, (20000, 16385)),  # more than 64 chunks of 256 keys
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}/{c[2]}x{c[3]}x{c[4]}{'bf16' if c[5] else 'f32'}"
                                              + ("_ragged" if c[6] else "") for c in CASES])
def test_attn_decode_shapes(case):
    B, Hq, Hkv, S, D, bf16, choices = case
    q, k, v, L = synth.attn_decode_inputs(B, Hq, Hkv, S, D, seed=6100 + S + D, choices=choices, bf16=bf16)
    if choices is not None:
        L = np.asarray([choices[i % len(choices)] for i in range(B)], dtype=np.int32)
        q, k, v, L = synth.attn_decode_inputs(B, Hq, Hkv, S, D, seed=6100 + S + D, lengths=L, bf16=bf16)
    got, lse = run(q, k, v, lengths=L, bf16=bf16)
    compare(q, k, v, got, lse, lengths=L, bf16=bf16, what=str(case))


def test_attn_decode_lengths_beyond_range_and_empty():
    """Lengths are clamped to [0, S]; an empty key set gives o = 0, lse = -inf;
    with no keys at all (S = 0) every row is empty."""
    B, Hq, Hkv, S, D = 4, 4, 2, 300, 128
    L = np.array([-5, 0, 299, 10**6], dtype=np.int32)
    q, k, v, _ = synth.attn_decode_inputs(B, Hq, Hkv, S, D, seed=6200, lengths=np.clip(L, 0, S), bf16=True)
    got, lse = run(q, k, v, lengths=L)
    compare(q, k, v, got, lse, lengths=L, what="clamped lengths")
    assert np.all(got[:2] == 0) and np.all(np.isneginf(lse[:2]))
    q0 = q[:, :, :]
    k0 = np.zeros((B, Hkv, 0, D), dtype=np.uint16)
    got0, lse0 = run(q0, k0, k0)
    assert np.all(got0 == 0) and np.all(np.isneginf(lse0))


def test_attn_decode_scale_and_without_lse():
    q, k, v, _ = synth.attn_decode_inputs(2, 8, 4, 520, 128, seed=6300, bf16=True)
    got, _ = run(q, k, v, scale=0.37, want_lse=False)
    compare(q, k, v, got, None, scale=0.37, what="scale 0.37")


def test_attn_decode_nan_row():
    """A NaN inside the valid keys makes that row NaN (both heads of its group)."""
    q, k, v, _ = synth.attn_decode_inputs(2, 4, 2, 300, 64, seed=6400, bf16=False)
    k[1, 0, 123, 5] = np.nan
    got, lse = run(q, k, v, bf16=False)
    assert np.all(np.isnan(got[1, :2])) and np.all(np.isnan(lse[1, :2]))
    assert not np.isnan(got[0]).any() and not np.isnan(got[1, 2:]).any()
    compare(q, k, v, got, lse, bf16=False, what="NaN row")


def test_attn_decode_benchmark_shape_and_determinism():
    """The measured workload in full: batch 8, 32 query heads on 8 key-value
    heads, 8192 keys, dim 128, bf16; and the same bits on a second run."""
    q, k, v, _ = synth.attn_decode_inputs(8, 32, 8, 8192, 128, seed=6001, bf16=True)
    got, lse = run(q, k, v)
    compare(q, k, v, got, lse, what="8x32/8x8192x128 bf16")
    got2, lse2 = run(q, k, v)
    assert np.array_equal(got, got2) and np.array_equal(lse, lse2)
