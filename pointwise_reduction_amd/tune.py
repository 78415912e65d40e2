"""Selection of launch configurations on the target GPU ("Stax (4): GPU
Codegen and Dynamic Shapes", 9.6).

    python -m pointwise_reduction_amd.tune [--workload NAME ...] [--steps K] [--reps R]
                                           [--search] [--cache PATH] [--q Q --delta D]

Without --search: Algorithm 9.1 over each workload's small candidate set of
(form, launch knobs); candidates without a compiled kernel, or that cannot
serve the shape, count as infinitely slow; the fastest is reported. The
planner's constants (fr_plan.cpp) hold the winners measured this way.

With --search, the full procedure:
  1. the cache (Algorithm 9.1, lines 1 and 7): a record for the same kernel
     sources (SHA-256 of csrc/), operation, shape, dtype and candidate set is
     used as is, without measuring;
  2. otherwise Algorithm 9.1 over the candidate set;
  3. the timing noise eta_max of the best candidate, from repeated replays,
     and eps = fr_tune_threshold(eta_max) > 2 eta_max / (1 + eta_max) (the
     remark after Proposition 9.2);
  4. random search over the workload's configuration space (Definition 9.2)
     with N = fr_tune_random_draws(q, delta) draws (Proposition 9.3: 60 for
     q = delta = 0.05);
  5. coordinate descent (Algorithm 9.2) from the better of 2 and 4;
  6. the winner is recorded in the library for this exact shape
     (fr_tune_record) and in the cache file.
load_cache() records every cached winner for the current sources, so later
calls of those shapes in the process use them.

Each configuration runs through the C ABI with fr_tune_override, over buffer
sets that rotate through >= 1 GiB so reads come from HBM, as K graph-replayed
steps; the median of R replays is its time. Its output must match the
automatic plan's output (to the tolerances of the parity tests) or its time
is infinite: a configuration that computes something else is never chosen.
"""
import argparse
import hashlib
import json
import math
import os
import sys

import numpy as np
import torch

import pointwise_reduction_amd as fr
from pointwise_reduction_amd import timing

ROTATE_BYTES = 1 << 30


def _sets(per_set):
    return max(2, math.ceil(ROTATE_BYTES / per_set))


def _d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bf(u):
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).cuda().view(torch.bfloat16)


def workload(name):
    """(op, logical bytes, per-set bytes, alloc(sets) -> launch(k), output(), candidates)."""
    import synth
    P, R, S = fr.FR_FORM_PER, fr.FR_FORM_RED, fr.FR_FORM_SPLIT
    if name == "softmax":
        rows, cols = 4096, 1024
        x = synth.softmax_inputs(rows, cols, seed=2001)
        cands = [dict(form=P, threads=256, seg=64, vec=4, rows_per_wg=4),
                 dict(form=P, threads=256, seg=64, vec=4, rows_per_wg=8),
                 dict(form=P, threads=256, seg=64, vec=4, rows_per_wg=16),
                 dict(form=P, threads=256, seg=32, vec=8, rows_per_wg=8),
                 dict(form=P, threads=256, seg=32, vec=8, rows_per_wg=16),
                 dict(form=R, threads=256, vec=4), dict(form=R, threads=512, vec=2)]

        def alloc(sets):
            xs = [_d(x) for _ in range(sets)]
            ys = [torch.empty_like(xs[0]) for _ in range(sets)]
            return (lambda k: fr.fr_softmax_rows(xs[k], ys[k])), (lambda: ys[0])
        return fr.FR_OP_SOFTMAX, 8 * rows * cols, 8 * rows * cols, alloc, cands, "f32"
    if name == "add_2d":
        n = 8192
        x = synth.normal((n, n), 62, stream=1)
        y = synth.normal((n, n), 62, stream=2)
        PW = fr.FR_FORM_POINTWISE
        cands = [dict(form=PW, threads=256, rows_per_wg=ti, chunk=tj, grid=g)
                 for ti, tj in ((64, 64), (32, 128), (128, 32), (64, 128), (128, 64), (32, 32))
                 for g in (0, 2048)]

        def alloc(sets):
            xs = [_d(x) for _ in range(sets)]
            ys = [_d(y) for _ in range(sets)]
            outs = [torch.empty_like(ys[0]) for _ in range(sets)]
            return (lambda k: fr.fr_add_2d(xs[k].t(), ys[k], outs[k])), (lambda: outs[0])
        return fr.FR_OP_ADD_2D, 12 * n * n, 12 * n * n, alloc, cands, "exact"
    if name == "gelu_bwd":
        n = 1 << 28
        h = synth.normal((n,), 54, stream=3, std=2.0)
        PW = fr.FR_FORM_POINTWISE
        cands = [dict(form=PW, threads=256, vec=v, grid=g) for v in (1, 2, 4) for g in (0, 1024, 4096)]

        def alloc(sets):
            hs = [_d(h) for _ in range(sets)]
            g = torch.tensor([0.5], dtype=torch.float32, device="cuda")
            outs = [torch.empty_like(hs[0]) for _ in range(sets)]
            return (lambda k: fr.fr_gelu_backward(g, hs[k], outs[k])), (lambda: outs[0])
        return fr.FR_OP_GELU_BWD, 8 * n, 8 * n, alloc, cands, "f32row"
    if name == "softmax_bwd":
        rows, cols = 4096, 1024
        y = synth.softmax_inputs(rows, cols, seed=2001)  # any fp32 rows serve as y for timing
        g = synth.normal((rows, cols), 2001, stream=7)
        cands = [dict(form=P, threads=256, seg=64, vec=4, rows_per_wg=4),
                 dict(form=P, threads=256, seg=64, vec=4, rows_per_wg=8),
                 dict(form=R, threads=256, vec=4), dict(form=R, threads=512, vec=2)]

        def alloc(sets):
            ys = [_d(y) for _ in range(sets)]
            gs = [_d(g) for _ in range(sets)]
            xs = [torch.empty_like(ys[0]) for _ in range(sets)]
            return (lambda k: fr.fr_softmax_rows_backward(ys[k], gs[k], xs[k])), (lambda: xs[0])
        return fr.FR_OP_SOFTMAX_BWD, 12 * rows * cols, 12 * rows * cols, alloc, cands, "f32row"
    if name == "ragged":
        rows, cap = 512, 131072
        x, L = synth.ragged_softmax_inputs(rows, cap, seed=5001)
        nbytes = 8 * int(L.sum()) + 8 * rows
        cands = [dict(form=S, threads=256, vec=8, passes=p) for p in (1, 2)]
        cands += [dict(form=S, threads=256, vec=4, passes=p) for p in (1, 2)]
        cands += [dict(form=S, threads=512, vec=4, passes=p) for p in (1, 2)]
        cands += [dict(form=S, threads=256, vec=8, passes=1, wait_us=w) for w in (20, 1000)]
        cands += [dict(form=R, threads=512, vec=2), dict(form=R, threads=1024, vec=2)]

        def alloc(sets):
            Ld = _d(L)
            xs = [_d(x) for _ in range(sets)]
            ys = [torch.empty_like(xs[0]) for _ in range(sets)]
            ws = [fr.fr_softmax_rows_workspace_init(torch.empty((rows * 64 * 16 + 4096) // 4, dtype=torch.float32,
                                                                device="cuda")) for _ in range(sets)]
            am = [torch.empty(rows, dtype=torch.int32, device="cuda") for _ in range(sets)]
            return (lambda k: fr.fr_softmax_rows(xs[k], ys[k], lengths=Ld, argmax=am[k], ws=ws[k])), \
                (lambda: ys[0].masked_fill(torch.arange(cap, device="cuda")[None, :] >= Ld[:, None].long(), 0))
        return fr.FR_OP_SOFTMAX, nbytes, 8 * rows * cap, alloc, cands, "f32"
    if name == "layernorm":
        rows, cols = 2048, 32768
        x, g, b = synth.layernorm_inputs(rows, cols, seed=3001)
        cands = [dict(form=P, threads=512, vec=8), dict(form=P, threads=1024, vec=4),
                 dict(form=P, threads=512, vec=8, rows_per_wg=8), dict(form=P, threads=512, vec=8, rows_per_wg=6),
                 dict(form=P, threads=512, vec=8, rows_per_wg=5), dict(form=P, threads=512, vec=8, rows_per_wg=4),
                 dict(form=P, threads=512, vec=8, rows_per_wg=3),
                 dict(form=R, threads=256, vec=4), dict(form=R, threads=512, vec=2), dict(form=R, threads=1024, vec=2)]

        def alloc(sets):
            gd, bd = _bf(g), _bf(b)
            xs = [_bf(x) for _ in range(sets)]
            ys = [torch.empty_like(xs[0]) for _ in range(sets)]
            return (lambda k: fr.fr_layernorm_rows(xs[k], ys[k], gamma=gd, beta=bd)), (lambda: ys[0])
        return fr.FR_OP_LAYERNORM, 4 * rows * cols + 4 * cols, 4 * rows * cols, alloc, cands, "bf16"
    if name == "sumsq":
        n = 1 << 28
        x = synth.sumsq_inputs(n, seed=4001)
        cands = [dict(form=S, threads=256, vec=4, chunk=c) for c in (1 << 15, 1 << 16, 1 << 17, 1 << 18)]
        cands += [dict(form=S, threads=256, vec=8, chunk=1 << 17), dict(form=S, threads=512, vec=2, chunk=1 << 17)]

        def alloc(sets):
            xs = [_d(x) for _ in range(sets)]
            outs = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(sets)]
            ws = [torch.empty(1 << 14, dtype=torch.float32, device="cuda") for _ in range(sets)]
            return (lambda k: fr.fr_sumsq_full(xs[k], outs[k], ws=ws[k])), (lambda: outs[0])
        return fr.FR_OP_SUMSQ, 4 * n + 4, 4 * n, alloc, cands, "f32"
    if name == "sum_relu_add":
        rows, cols = 64, 128
        a, b, _ = synth.sum_relu_add_inputs(rows, cols, seed=1001)
        cands = [dict(form=P, threads=256, seg=32, vec=1, rows_per_wg=8),
                 dict(form=P, threads=256, seg=64, vec=1, rows_per_wg=4),
                 dict(form=P, threads=256, seg=16, vec=2, rows_per_wg=16)]

        def alloc(sets):
            ad, bd = _d(a), _d(b)
            outs = [torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(sets)]
            return (lambda k: fr.fr_sum_relu_add(ad, bd, outs[k])), (lambda: outs[0])
        return fr.FR_OP_SUM_RELU_ADD, 8 * rows * cols + 4 * rows, 8 * rows * cols, alloc, cands, "f32"
    raise SystemExit(f"unknown workload {name}")


def search_space(name):
    """Definition 9.2 for one workload: (record key (op, rows, cols, dtype),
    parameter names, value sets, knobs(config) -> fr_tune_override knobs,
    config_of(knobs) -> config or None)."""
    P, R, S, PW = fr.FR_FORM_PER, fr.FR_FORM_RED, fr.FR_FORM_SPLIT, fr.FR_FORM_POINTWISE
    F32, BF16 = fr.FR_F32, fr.FR_BF16

    def pow2(lo, hi):
        return [1 << i for i in range(lo, hi + 1)]

    def per_rows(op, rows, cols):
        def knobs(c):
            seg, vec, rpw = c
            return dict(form=P, threads=256, seg=seg, vec=vec, rows_per_wg=256 // seg * rpw)

        def config_of(k):
            if k.get("form") != P:
                return None
            return (k["seg"], k["vec"], k["rows_per_wg"] * k["seg"] // 256)
        return (op, rows, cols, F32), ("seg", "vec", "rows_per_lane_group"), [pow2(3, 6), pow2(0, 3), pow2(0, 2)], \
            knobs, config_of
    if name == "softmax":
        return per_rows(fr.FR_OP_SOFTMAX, 4096, 1024)
    if name == "softmax_bwd":
        return per_rows(fr.FR_OP_SOFTMAX_BWD, 4096, 1024)
    if name == "sum_relu_add":
        return per_rows(fr.FR_OP_SUM_RELU_ADD, 64, 128)
    if name == "layernorm":
        def knobs(c):
            return dict(form=c[0], threads=c[1], vec=c[2])
        return (fr.FR_OP_LAYERNORM, 2048, 32768, BF16), ("form", "threads", "vec"), \
            [[P, R], pow2(6, 10), pow2(0, 3)], knobs, lambda k: (k["form"], k["threads"], k["vec"])
    if name == "add_2d":
        def knobs(c):
            return dict(form=PW, threads=256, rows_per_wg=c[0], chunk=c[1], grid=c[2])
        return (fr.FR_OP_ADD_2D, 8192, 8192, F32), ("tile_rows", "tile_cols", "grid"), \
            [pow2(4, 8), pow2(4, 8), pow2(10, 20)], knobs, \
            lambda k: (k["rows_per_wg"], k["chunk"], k["grid"] or (1 << 20))
    if name == "gelu_bwd":
        def knobs(c):
            return dict(form=PW, threads=256, vec=c[0], grid=c[1])
        return (fr.FR_OP_GELU_BWD, 1, 1 << 28, F32), ("vec", "grid"), [pow2(0, 2), pow2(9, 20)], knobs, \
            lambda k: (k["vec"], k["grid"] or (1 << 20))
    if name == "sumsq":
        def knobs(c):
            return dict(form=S, threads=c[0], vec=c[1], chunk=c[2])
        return (fr.FR_OP_SUMSQ, 1, 1 << 28, F32), ("threads", "vec", "chunk"), \
            [[256, 512], pow2(0, 3), pow2(14, 19)], knobs, lambda k: (k["threads"], k["vec"], k["chunk"])
    if name == "ragged":
        def knobs(c):
            return dict(form=S, passes=c[0], threads=c[1], vec=c[2], wait_us=c[3])
        return (fr.FR_OP_SOFTMAX, 512, 131072, F32), ("passes", "threads", "vec", "wait_us"), \
            [[1, 2], [256, 512], [2, 4, 8], [25, 50, 100, 200, 400, 800]], knobs, \
            lambda k: None if k.get("form") != S else (k.get("passes", 1), k["threads"], k["vec"],
                                                        k.get("wait_us") or 200)
    raise SystemExit(f"no configuration space for workload {name}")


def source_hash():
    """SHA-256 of the kernel sources: a cached selection holds while they do
    not change (Algorithm 9.1 keys its record by the kernel source)."""
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def default_cache_path():
    return os.environ.get("FR_TUNE_CACHE") or os.path.join(os.path.expanduser("~"), ".cache",
                                                           "pointwise_reduction_amd", "tune_cache.json")


def _read_cache(path):
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def _write_cache(path, cache):
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(cache, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


def _cache_key(src, key, cands):
    op, rows, cols, dtype = key
    c = hashlib.sha256(json.dumps(cands, sort_keys=True).encode()).hexdigest()[:16]
    return f"{src[:16]}:op{op}:{rows}x{cols}:dt{dtype}:C{c}"


def load_cache(path=None):
    """Record every cached selection made for the current kernel sources
    (fr_tune_record); returns how many were recorded."""
    src = source_hash()[:16]
    n = 0
    for k, v in _read_cache(path or default_cache_path()).items():
        if k.startswith(src + ":"):
            op, rows, cols, dtype = v["key"]
            fr.fr_tune_record(op, rows, cols, dtype, **v["knobs"])
            n += 1
    return n


def search(name, steps, reps, q=0.05, delta=0.05, seed=1, cache_path=None, log=print):
    """The full procedure of the module docstring for one workload."""
    op, nbytes, per_set, alloc, cands, kind = workload(name)
    key, names, value_sets, knobs_of, config_of = search_space(name)
    assert key[0] == op
    cache_path = cache_path or default_cache_path()
    src = source_hash()
    ckey = _cache_key(src, key, cands)
    cache = _read_cache(cache_path)
    if ckey in cache:
        hit = cache[ckey]
        fr.fr_tune_record(*key, **hit["knobs"])
        log(f"  {name}: cached selection {hit['knobs']} ({hit['ms_per_step'] * 1000:.3f} us), not measured")
        return dict(hit, cached=True)

    sets = min(_sets(per_set), steps)
    launch, output = alloc(sets)
    fr.fr_tune_override(op)
    launch(0)
    torch.cuda.synchronize()
    ref = output().clone()
    memo = {}

    def measure(kn, r=reps):
        mk = tuple(sorted(kn.items()))
        if mk in memo:
            return memo[mk]
        try:
            fr.fr_tune_override(op, **kn)
            launch(0)
            torch.cuda.synchronize()
            if not close(output(), ref, kind):
                t = math.inf
            else:
                graph = timing.capture(lambda k: launch(k % sets), steps)
                t = float(np.median(timing.time_replays(graph, steps, r)))
                del graph
        except fr.FrError:  # no compiled kernel, or the knobs cannot serve this shape
            t = math.inf
        finally:
            fr.fr_tune_override(op)
        memo[mk] = t
        return t

    # Algorithm 9.1 over the candidate set
    cand_t = [(measure(c), c) for c in cands]
    t_c, best_c = min(cand_t, key=lambda x: x[0])
    log(f"  {name}: Algorithm 9.1 over {len(cands)} candidates: {best_c} {t_c * 1000:.3f} us")
    # timing noise of that configuration, and the descent threshold
    fr.fr_tune_override(op, **best_c)
    graph = timing.capture(lambda k: launch(k % sets), steps)
    ts = timing.time_replays(graph, steps, max(reps, 8))
    del graph
    fr.fr_tune_override(op)
    med = float(np.median(ts))
    eta = max(abs(t / med - 1.0) for t in ts)
    eps = fr.fr_tune_threshold(min(eta, 0.5))
    # random search over the whole space
    n_draws = fr.fr_tune_random_draws(q, delta)
    cost = lambda c: measure(knobs_of(c))  # noqa: E731
    try:
        r_cfg, r_res = fr.fr_tune_random_search(value_sets, n_draws, seed, cost)
        t_r = r_res.cost
    except fr.FrError:
        r_cfg, t_r = None, math.inf
    log(f"  {name}: eta_max {eta:.4f} -> eps {eps:.4f}; random search, {n_draws} draws "
        f"(q={q}, delta={delta}): {dict(zip(names, r_cfg)) if r_cfg else None} {t_r * 1000:.3f} us")
    # coordinate descent from the better start
    c_cfg = config_of(best_c)
    starts = [(t_r, r_cfg)] + ([(t_c, c_cfg)] if c_cfg is not None and
                               all(v in s for v, s in zip(c_cfg, value_sets)) else [])
    t0, start = min((x for x in starts if x[1] is not None), key=lambda x: x[0], default=(math.inf, None))
    if start is not None and t0 < math.inf:
        d_cfg, d_res = fr.fr_tune_coordinate_descent(value_sets, start, eps, cost)
        final_kn, t_f = knobs_of(d_cfg), d_res.cost
        log(f"  {name}: coordinate descent from {dict(zip(names, start))}: {dict(zip(names, d_cfg))} "
            f"{t_f * 1000:.3f} us ({d_res.accepted} accepted, {d_res.rounds} rounds)")
    else:
        final_kn, t_f = best_c, t_c
    if t_c < t_f:  # a candidate outside the space can still win
        final_kn, t_f = best_c, t_c
    out = {"workload": name, "key": list(key), "knobs": final_kn, "ms_per_step": t_f,
           "GB/s": round(nbytes / (t_f * 1e-3) / 1e9, 1), "eta_max": eta, "eps": eps,
           "measured": len(memo), "candidates_best": {"knobs": best_c, "ms_per_step": t_c}}
    fr.fr_tune_record(*key, **final_kn)
    cache[ckey] = out
    _write_cache(cache_path, cache)
    log(f"  {name}: selected {final_kn} {t_f * 1000:.3f} us ({out['GB/s']} GB/s), {len(memo)} configurations "
        f"measured; recorded for {key[1]}x{key[2]}")
    return dict(out, cached=False)


def close(a, b, kind):
    a = a.float().cpu().numpy().astype(np.float64)
    b = b.float().cpu().numpy().astype(np.float64)
    if kind == "bf16":
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -126))) - 7)
        return bool(np.all(np.abs(a - b) <= 2 * ulp + 1e-6))
    if kind == "exact":
        return bool(np.array_equal(a, b))
    if kind == "f32row":  # differences of products cancel: scale by the row's largest value
        scale = np.max(np.abs(b), axis=-1, keepdims=True)
        return bool(np.all(np.abs(a - b) <= 2e-5 * scale + 2e-6))
    return bool(np.all(np.abs(a - b) <= 2e-5 * np.abs(b) + 2e-6))


def tune(name, steps, reps):
    op, nbytes, per_set, alloc, cands, kind = workload(name)
    sets = min(_sets(per_set), steps)
    launch, output = alloc(sets)
    fr.fr_tune_override(op)
    launch(0)
    torch.cuda.synchronize()
    ref = output().clone()
    results = []
    for cand in [None] + cands:
        label = "auto" if cand is None else ",".join(f"{k}={v}" for k, v in cand.items())
        try:
            if cand is not None:
                fr.fr_tune_override(op, **cand)
            launch(0)
            torch.cuda.synchronize()
            ok = close(output(), ref, kind)
            graph = timing.capture(lambda k: launch(k % sets), steps)
            ms = float(np.median(timing.time_replays(graph, steps, reps)))
            del graph
        except fr.FrError as e:  # no compiled kernel, shape does not fit: t = infinity
            ok, ms = False, math.inf
            label += f" ({fr.status_string(e.status).split(':')[0]})"
        finally:
            fr.fr_tune_override(op)
        gbs = nbytes / (ms * 1e-3) / 1e9 if ms != math.inf else 0.0
        results.append({"candidate": label, "ms_per_step": ms, "GB/s": round(gbs, 1), "matches_auto": ok})
        print(f"  {name:13s} {label:60s} {ms * 1000:9.3f} us {gbs:8.1f} GB/s {'ok' if ok else 'MISMATCH'}",
              flush=True)
    valid = [r for r in results if r["matches_auto"] and r["ms_per_step"] != math.inf]
    best = min(valid, key=lambda r: r["ms_per_step"]) if valid else None
    return {"workload": name, "sets": sets, "steps": steps, "best": best, "results": results}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", nargs="*", default=["softmax", "ragged", "layernorm", "sumsq", "sum_relu_add"])
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--json", default=None, help="write the full table here")
    ap.add_argument("--search", action="store_true",
                    help="cache, candidates, noise, random search and coordinate descent (see above)")
    ap.add_argument("--cache", default=None, help="cache file (default $FR_TUNE_CACHE or ~/.cache/...)")
    ap.add_argument("--q", type=float, default=0.05)
    ap.add_argument("--delta", type=float, default=0.05)
    ap.add_argument("--seed", type=int, default=1)
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    torch.cuda.set_device(0)
    if args.search:
        out = [search(w, args.steps, args.reps, args.q, args.delta, args.seed, args.cache) for w in args.workload]
        if args.json:
            with open(args.json, "w") as f:
                json.dump(out, f, indent=1)
        return
    out = [tune(w, args.steps, args.reps) for w in args.workload]
    for t in out:
        b = t["best"]
        print(f"best {t['workload']}: {b['candidate'] if b else None} "
              f"{b['ms_per_step'] * 1000 if b else float('nan'):.3f} us")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
