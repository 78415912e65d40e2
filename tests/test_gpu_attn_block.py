"""GPU parity: tiled attention over blocks of query rows against the fp64
oracle ("Stax (4)", 9.10; causal mask of Listing 9.7; the pages' sizes
N = 256 and 300, causal and not, and N = 4096, d = 128).

bf16 q, k, v ~ N(0, 1). Both products run on the matrix cores with fp32
accumulation; P enters the second product as two bf16 parts (its rounding
and the rounding of the remainder), so it carries about fp32 accuracy. o is
held to the rule of every bf16 output: within one bf16 ulp of the oracle's
bf16 value, or - a near-cancellation - within the fp32 rule on its terms,
1e-5 * sum_j p_j |v_jd| + 1e-6; lse within 1e-5 * (1 + max_j sum_d
|scale q_d k_jd|) (the fp32 rule on the scores' terms).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_of, bf16_bits_tensor, bf16_to_f64, check_bf16, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402


def run(qb, kb, vb, causal, scale=None):
    """Returns (o as bf16 bit patterns, lse)."""
    q, k, v = bf16_bits_tensor(qb), bf16_bits_tensor(kb), bf16_bits_tensor(vb)
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fr.fr_attn_block(q, k, v, o, lse, causal=causal, scale=scale)
    return bf16_bits_of(o), host(lse)


def check(o_bits, lse, o64, lse64, mag, smag, what):
    check_bf16(o_bits, oracle.round_bf16(o64), o64, mag, what=what)
    okl = np.abs(lse - lse64) <= 1e-5 * (1 + smag)
    assert okl.all(), f"{what}: lse off by {np.abs(lse - lse64).max():.3e}"


CASES = [  # B, Hq, Hkv, Nq, Nk, D
    (1, 1, 1, 256, 256, 64), (1, 1, 1, 300, 300, 64), (1, 2, 1, 300, 300, 128), (2, 4, 2, 129, 129, 128),
    (1, 2, 2, 1, 1, 64), (1, 1, 1, 64, 64, 128), (1, 2, 1, 200, 333, 128), (1, 2, 1, 333, 200, 64),
    (2, 8, 2, 512, 512, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_attn_block(case, causal):
    B, Hq, Hkv, Nq, Nk, D = case
    qb, kb, vb = synth.attn_block_inputs(B, Hq, Hkv, Nq, Nk, D, seed=7000 + Nq + Nk + D)
    o, lse = run(qb, kb, vb, causal)
    o64, lse64, mag, smag = oracle.attn_fwd(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), causal=causal)
    check(o, lse, o64, lse64, mag, smag, f"{case} causal={causal}")


def test_attn_block_scale_and_empty_keys():
    qb, kb, vb = synth.attn_block_inputs(1, 2, 2, 130, 70, 64, seed=7101)
    o, lse = run(qb, kb, vb, False, scale=0.3)
    o64, lse64, mag, smag = oracle.attn_fwd(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), scale=0.3)
    check(o, lse, o64, lse64, mag, smag, "scale 0.3")
    q = torch.zeros((1, 1, 5, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.zeros((1, 1, 5), dtype=torch.float32, device="cuda")
    fr.fr_attn_block(q, kv, kv, o, lse)
    assert np.all(host(o.float()) == 0.0) and np.all(np.isneginf(host(lse)))


def test_attn_block_argument_errors():
    q = torch.zeros((1, 3, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 3, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(fr.FrError) as ei:
        fr.fr_attn_block(q, k, k, torch.empty_like(q), lse)  # 3 query heads on 2 key-value heads
    assert ei.value.status == fr.FR_E_ARG
    q2 = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda")
    k2 = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fr.FrError) as ei:
        fr.fr_attn_block(q2, k2, k2, torch.empty_like(q2), torch.zeros((1, 2, 8), device="cuda"))
    assert ei.value.status == fr.FR_E_SIZE


@pytest.mark.parametrize("causal", [True, False])
def test_attn_block_full_size_sampled(causal):
    # 4 x 16 heads x 4096 x 128, the benchmark's launch; rows sampled, each
    # checked against the oracle's decode row over the keys it may see
    B, H, N, D = 4, 16, 4096, 128
    qb, kb, vb = synth.attn_block_inputs(B, H, H, N, N, D, seed=7001)
    o, lse = run(qb, kb, vb, causal)
    rng = np.random.default_rng(11)
    for _ in range(12):
        b, h, i = int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))
        L = np.array([i + 1 if causal else N], np.int32)
        od, ld, mag, smag = oracle.attn_decode(bf16_to_f64(qb[b:b + 1, h:h + 1, i]), bf16_to_f64(kb[b:b + 1, h:h + 1]),
                                               bf16_to_f64(vb[b:b + 1, h:h + 1]), lengths=L)
        check(o[b, h, i], lse[b, h, i], od[0, 0], ld[0, 0], mag[0, 0], smag[0, 0], f"b{b} h{h} i{i}")
