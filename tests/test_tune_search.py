"""The configuration search core ("Stax (4)", 9.6) on the CPU.

Deterministic synthetic cost tables stand in for measured times, so the
statements of the pages can be checked exactly: Algorithm 9.2 ends at a point
no single doubling or halving improves by more than eps, after at most
min(|Pi|, ceil(log(t0/tmin) / -log(1 - eps))) acceptances (Proposition 9.2);
under relative noise |eta| <= eta_max with eps above 2 eta/(1 + eta) every
accepted move is a real improvement; the best of N uniform draws lies in the
fastest q-fraction with probability >= 1 - (1 - q)^N (Proposition 9.3).
"""
import itertools
import math

import numpy as np
import pytest

import pointwise_reduction_amd as fr

SPACE = [[1, 2, 4, 8, 16, 32], [64, 128, 256, 512, 1024], [1, 2, 4, 8]]


def table(seed, inf_frac=0.15):
    rng = np.random.default_rng(seed)
    t = {c: float(rng.lognormal(0.0, 0.6)) for c in itertools.product(*SPACE)}
    for c in list(t):
        if rng.random() < inf_frac:
            t[c] = math.inf
    return t


def neighbours(c):
    for i, v in enumerate(c):
        for w in (v * 2, v // 2 if v % 2 == 0 else None):
            if w is not None and w in SPACE[i]:
                yield c[:i] + (w,) + c[i + 1:]


def test_draws_and_threshold_formulas():
    assert fr.fr_tune_random_draws(0.05, 0.05) == 60  # the pages' example
    assert fr.fr_tune_random_draws(0.1, 0.01) == math.ceil(math.log(100) / 0.1)
    assert fr.fr_tune_random_draws(1.0, 0.5) == 1
    with pytest.raises(fr.FrError):
        fr.fr_tune_random_draws(0.0, 0.05)
    for eta in (0.0, 1e-4, 0.005, 0.01, 0.2):
        eps = fr.fr_tune_threshold(eta)
        assert eps > 2 * eta / (1 + eta) and eps >= 1e-3 and eps < 2 * eta / (1 + eta) + 1.1e-3
    assert fr.fr_tune_threshold(-0.1) == -1.0 and fr.fr_tune_threshold(1.0) == -1.0


@pytest.mark.parametrize("seed", range(12))
def test_coordinate_descent_local_optimum_and_acceptance_bound(seed):
    t = table(seed)
    calls = []

    def cost(c):
        calls.append(c)
        return t[c]
    finite = [c for c in t if t[c] < math.inf]
    start = finite[seed % len(finite)]
    eps = 1e-3
    c, res = fr.fr_tune_coordinate_descent(SPACE, start, eps, cost)
    assert res.cost == t[c] and t[c] <= t[start]
    for n in neighbours(c):  # Proposition 9.2: no neighbour is better by more than eps
        assert t[n] >= (1 - eps) * t[c]
    tmin = min(finite, key=t.get)
    bound = min(len(t), math.ceil(math.log(t[start] / t[tmin]) / -math.log(1 - eps)) if t[start] > t[tmin] else 0)
    assert res.accepted <= bound
    assert len(calls) == len(set(calls)) == res.evaluations  # each configuration measured once


@pytest.mark.parametrize("seed", range(8))
def test_coordinate_descent_under_bounded_noise(seed):
    # measured = true * (1 + eta_c), |eta_c| <= eta_max, fixed per configuration
    eta_max = 0.01
    t = table(100 + seed, inf_frac=0.0)
    rng = np.random.default_rng(seed)
    eta = {c: float(rng.uniform(-eta_max, eta_max)) for c in t}
    eps = fr.fr_tune_threshold(eta_max)
    path = []

    def cost(c):
        return t[c] * (1 + eta[c])
    start = list(t)[(seed * 37) % len(t)]
    c, res = fr.fr_tune_coordinate_descent(SPACE, start, eps, cost)
    # every acceptance lowers the true time, so the end is truly faster than
    # the start unless nothing was accepted; local optimality holds up to
    # eps + 2 eta_max
    if res.accepted:
        assert t[c] < t[start]
    for n in neighbours(c):
        assert t[n] >= (1 - eps - 2 * eta_max) * t[c] - 1e-12
    del path


def test_random_search_quantile_guarantee():
    # 1000 configurations with distinct times; N = 60 draws; the best lands
    # in the fastest 5% with probability >= 1 - 0.95^60 = 0.954
    space = [list(range(1, 11)), list(range(1, 11)), list(range(1, 11))]
    rng = np.random.default_rng(5)
    times = {c: float(v) for c, v in zip(itertools.product(*space), rng.permutation(1000) + 1)}
    q, n = 0.05, fr.fr_tune_random_draws(0.05, 0.05)
    hits = 0
    runs = 400
    for s in range(runs):
        c, res = fr.fr_tune_random_search(space, n, 1000 + s, times.get)
        assert res.cost == times[c] and res.evaluations <= n
        hits += times[c] <= q * 1000
    p = 1 - (1 - q) ** n
    assert hits / runs >= p - 4 * math.sqrt(p * (1 - p) / runs)


def test_random_search_draws_are_uniform():
    seen = {}

    def cost(c):
        seen[c] = seen.get(c, 0) + 1
        return 1.0
    space = [[1, 2, 3], [5, 7]]
    counts = np.zeros(6)
    for s in range(600):
        seen.clear()
        fr.fr_tune_random_search(space, 1, s, cost)
        (c,) = seen
        counts[[1, 2, 3].index(c[0]) * 2 + [5, 7].index(c[1])] += 1
    chi2 = float(((counts - 100) ** 2 / 100).sum())
    assert chi2 < 20.5  # 5 degrees of freedom, p ~ 0.001


def test_search_argument_errors():
    f = lambda c: 1.0  # noqa: E731
    with pytest.raises(fr.FrError):
        fr.fr_tune_coordinate_descent(SPACE, (3, 64, 1), 1e-3, f)  # start outside the space
    with pytest.raises(fr.FrError):
        fr.fr_tune_coordinate_descent(SPACE, (1, 64, 1), 0.0, f)
    with pytest.raises(fr.FrError):
        fr.fr_tune_coordinate_descent(SPACE, (1, 64, 1), 1e-3, lambda c: math.inf)
    with pytest.raises(fr.FrError):
        fr.fr_tune_random_search(SPACE, 10, 1, lambda c: math.inf)
    with pytest.raises(ZeroDivisionError):
        fr.fr_tune_random_search(SPACE, 10, 1, lambda c: 1 / 0)


def test_records_are_used_by_the_planner_for_that_shape_only():
    fr.fr_tune_clear()
    try:
        base = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024)
        assert fr.fr_tune_lookup(fr.FR_OP_SOFTMAX, 4096, 1024) is None
        fr.fr_tune_record(fr.FR_OP_SOFTMAX, 4096, 1024, fr.FR_F32, form=fr.FR_FORM_PER, threads=256, seg=32,
                          vec=8, rows_per_wg=16)
        p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024)
        assert (p.seg, p.vec, p.rows_per_wg) == (32, 8, 16) != (base.seg, base.vec, base.rows_per_wg)
        other = fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1000)  # another shape: defaults
        assert (other.seg, other.vec) == (base.seg, base.vec)
        assert fr.fr_tune_lookup(fr.FR_OP_SOFTMAX, 4096, 1024).seg == 32
        fr.fr_tune_record(fr.FR_OP_SOFTMAX, 4096, 1024, fr.FR_F32)  # remove
        assert fr.fr_plan_query(fr.FR_OP_SOFTMAX, 4096, 1024).seg == base.seg
    finally:
        fr.fr_tune_clear()


def test_cache_records_only_entries_of_the_current_sources(tmp_path):
    import json

    from pointwise_reduction_amd import tune
    fr.fr_tune_clear()
    src = tune.source_hash()
    knobs = dict(form=fr.FR_FORM_POINTWISE, threads=256, rows_per_wg=32, chunk=128, grid=0)
    key = [fr.FR_OP_ADD_2D, 1024, 2048, fr.FR_F32]
    cache = {tune._cache_key(src, key, []): {"key": key, "knobs": knobs, "ms_per_step": 0.1},
             tune._cache_key("0" * 64, key[:2] + [4096, 0], []): {"key": key[:2] + [4096, 0], "knobs": knobs,
                                                               "ms_per_step": 0.1}}
    path = tmp_path / "cache.json"
    path.write_text(json.dumps(cache))
    try:
        assert tune.load_cache(str(path)) == 1
        p = fr.fr_plan_query(fr.FR_OP_ADD_2D, 1024, 2048)
        assert (p.rows_per_wg, p.chunk) == (32, 128)
        assert fr.fr_tune_lookup(fr.FR_OP_ADD_2D, 1024, 4096) is None  # stale sources: not recorded
    finally:
        fr.fr_tune_clear()


def test_every_search_space_holds_the_planner_default():
    # the planner's measured default for each workload's shape is a point of
    # that workload's configuration space (so the search can only improve on it)
    from pointwise_reduction_amd import tune
    for name in ("softmax", "softmax_bwd", "sum_relu_add", "layernorm", "add_2d", "gelu_bwd", "sumsq"):
        (op, rows, cols, dtype), names, sets, knobs_of, config_of = tune.search_space(name)
        if name == "sumsq":  # a full reduction always takes the split form
            prev = fr.fr_force_form(fr.FR_FORM_SPLIT)
            try:
                p = fr.fr_plan_query(op, rows, cols, dtype=dtype, ws_bytes=1 << 30)
            finally:
                fr.fr_force_form(prev)
        else:
            p = fr.fr_plan_query(op, rows, cols, dtype=dtype)
        kn = {k: getattr(p, k) for k in ("form", "threads", "seg", "vec", "rows_per_wg", "chunk", "grid")}
        if name == "add_2d":
            kn["grid"] = 0
        if name == "gelu_bwd":
            kn["grid"] = 0
        cfg = config_of(kn)
        assert cfg is not None and all(v in s for v, s in zip(cfg, sets)), (name, kn, cfg)
