"""GPU: the configuration search ("Stax (4)", 9.6) end to end.

A recorded selection changes the launch of exactly its shape and the
results stay those of the oracle; the full search (Algorithm 9.1 over the
candidates, random search, coordinate descent) on the Example 1.1 sums
records a selection and caches it, and a second search with the same kernel
sources takes the cached record without measuring.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_fp32, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import pointwise_reduction_amd as fr  # noqa: E402
from pointwise_reduction_amd import tune  # noqa: E402


def test_recorded_selection_is_used_and_correct():
    x = synth.softmax_inputs(256, 1000, seed=2001)
    y64, _ = oracle.softmax_rows(x)
    fr.fr_tune_clear()
    try:
        for knobs in (dict(form=fr.FR_FORM_PER, threads=256, seg=64, vec=4, rows_per_wg=4),
                      dict(form=fr.FR_FORM_RED, threads=512, vec=2)):
            fr.fr_tune_record(fr.FR_OP_SOFTMAX, 256, 1000, fr.FR_F32, **knobs)
            assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 256, 1000).form == knobs["form"]
            y = torch.empty((256, 1000), dtype=torch.float32, device="cuda")
            fr.fr_softmax_rows(dev(x), y)
            check_fp32(host(y), y64, terms=None, what=str(knobs))
    finally:
        fr.fr_tune_clear()


def test_search_records_and_caches(tmp_path):
    fr.fr_tune_clear()
    cache = str(tmp_path / "tune.json")
    lines = []
    try:
        first = tune.search("sum_relu_add", steps=20, reps=3, cache_path=cache, log=lines.append)
        assert not first["cached"] and first["ms_per_step"] < float("inf")
        rec = fr.fr_tune_lookup(fr.FR_OP_SUM_RELU_ADD, 64, 128)
        assert rec is not None and rec.form == first["knobs"]["form"]
        assert first["measured"] >= 7  # at least the candidate set was measured
        fr.fr_tune_clear()
        second = tune.search("sum_relu_add", steps=20, reps=3, cache_path=cache, log=lines.append)
        assert second["cached"] and second["knobs"] == first["knobs"]
        assert fr.fr_tune_lookup(fr.FR_OP_SUM_RELU_ADD, 64, 128) is not None
        # the selection computes Example 1.1 correctly
        a, b, _ = synth.sum_relu_add_inputs(64, 128, seed=1001)
        out = torch.empty(64, dtype=torch.float32, device="cuda")
        fr.fr_sum_relu_add(dev(a), dev(b), out)
        _, ref = oracle.sum_relu_add(a, b)
        check_fp32(host(out), ref, what="selected configuration")
    finally:
        fr.fr_tune_clear()
    assert any("random search" in s for s in lines) and any("coordinate descent" in s for s in lines)
