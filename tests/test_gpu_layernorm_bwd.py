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
    # 2048 x 32768 bf16 with gamma: the benchmark's launch. Column sums over
    # all rows against the oracle; dx on sampled rows.
    rows, cols = 2048, 32768
    x, dy, g, mean, rstd = inputs(rows, cols, seed=3001)
    got = run_bwd(x, dy, g, mean, rstd)
    ref = oracle.layernorm_backward_rows(x, dy, g, mean.astype(np.float64), rstd.astype(np.float64))
    check_fp32(got["dgamma"], ref["dgamma64"], terms=ref["gmag"], what="full dgamma")
    check_fp32(got["dbeta"], ref["dbeta64"], terms=ref["bmag"], what="full dbeta")
    rs = np.array([0, 1, 255, 256, 1023, 2047])
    check_bf16(got["dx"][rs], oracle.round_bf16(ref["dx64"][rs]), ref["dx64"][rs], ref["dxmag"][rs], what="full dx")
