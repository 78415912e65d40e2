"""Offline selection of launch configurations on the target GPU.

    python -m pointwise_reduction_amd.tune [--workload NAME ...] [--steps K] [--reps R]

Algorithm 9.1 of "Stax (4): GPU Codegen and Dynamic Shapes" (9.6) run ahead
of time: for each workload a small candidate set of (form, launch knobs) is
timed on the GPU, candidates without a compiled kernel count as infinitely
slow, and the fastest is reported. The winners are written into the
planner's constants (fr_plan.cpp) by hand; only spill-free kernels are
compiled (the build checks the compiler's resource report).

Each candidate runs through the C ABI with fr_tune_override, over buffer
sets that rotate through >= 1 GiB so reads come from HBM, as K graph-replayed
steps; the median of R replays is kept. Its output must match the automatic
plan's output (to the fp32 / bf16 tolerances used by the parity tests)
before its time counts.
"""
import argparse
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
            ws = [torch.empty((rows * 64 * 16 + 4096) // 4, dtype=torch.float32, device="cuda") for _ in range(sets)]
            am = [torch.empty(rows, dtype=torch.int32, device="cuda") for _ in range(sets)]
            return (lambda k: fr.fr_softmax_rows(xs[k], ys[k], lengths=Ld, argmax=am[k], ws=ws[k])), \
                (lambda: ys[0].masked_fill(torch.arange(cap, device="cuda")[None, :] >= Ld[:, None].long(), 0))
        return fr.FR_OP_SOFTMAX, nbytes, 8 * rows * cap, alloc, cands, "f32"
    if name == "layernorm":
        rows, cols = 2048, 32768
        x, g, b = synth.layernorm_inputs(rows, cols, seed=3001)
        cands = [dict(form=P, threads=512, vec=8), dict(form=P, threads=1024, vec=4),
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
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    torch.cuda.set_device(0)
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
