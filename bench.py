"""Benchmark of the fused row-reduction kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--warm] [--eager] [--procs N]
                    [--reps R]

A step is one pass of the whole operation over one batch of synthetic input
already resident in HBM. The default workload is the row softmax over
4096 x 1024 fp32 (the headline configuration). The other workloads are
selected with --workload: Example 1.1 sums, the softmax and its backward at
65536 rows and Example 1.1 at 2^20 rows (the largest shapes), LayerNorm
2048 x 32768 bf16 and at 8192 rows, the 2^28 sum of squares, the ragged 512-row softmax, decode and tiled attention,
softmax and LayerNorm backward, x.t() + y, GELU backward, a recorded region
of 16 Example 1.1 launches, and streaming references (copy, read, write,
and an empty kernel: the cost of one kernel boundary, reported in us per
step). Tiled attention reports TFLOP/s against the matrix cores' bf16 peak;
the others report GB/s against HBM.

Timing: W untimed steps, then exactly K steps between two events on the
launch stream, with a device synchronization on both sides. Consecutive
steps rotate through enough distinct buffer sets (>= 1 GiB in total) that
the 256 MB MALL cannot serve a step's reads from the previous use of the same
buffers (--warm uses one set). The K launches are captured once into a HIP
graph and replayed, so host launch overhead does not enter the device time
(--eager launches them one by one instead). The graph starts with an
untimed lead-in of whole rotations over the buffer sets (at least 256
steps), so every set is touched once between two uses whatever K is and the
device has been busy for a while when the first timed step starts; then a
device clock mark, the K timed steps
and a second mark. The marks enclose the K steps and one kernel boundary
more (the one after the first mark); a graph of the two marks alone behind
the same lead-in measures it (mark_interval_us), and the reported time is
the marks' difference less that interval: the device time of exactly the K
steps, each with its boundary to the next kernel. The marks' raw difference
is reported as marks_raw_ms_per_step, and events around a replay of the K
steps alone (behind a lead-in replay) as events_ms_per_step; the events
also hold a fixed cost of the graph's edges. The graph's output is checked
against an eager launch before the timing is reported.

The measurement runs in --procs N (default 3) separate processes, one after
the other; each times the K steps --reps R (default 3) times and reports the
median, and the line is the median process's (the median of medians), with
all N values and their range under "procs" ("hello-gpu, Chapter 12: Fusion",
12.5: medians over independent processes).

Output: one JSON line with the effective HBM bandwidth (logical bytes: each
input read once, each output written once), the roofline entry for the
dominant kernel and the fp64 oracle timed on the host (cpu_baseline).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PEAK_MFMA_BF16_TFS = 2500.0  # MI355X dense bf16 matrix-core peak
METRIC = "effective HBM GB/s and % of MI355X peak for fused reductions (softmax 4096x1024)"
ROTATE_BYTES = 1 << 30
LEAD_STEPS = 256  # at least this many lead-in steps, a whole number of rotations


# ------------------------------------------------------------------ logical bytes


def softmax_bytes(rows, cols, lengths=None, argmax=False):
    """Each valid input element read once and each output written once
    ("Stax (4)", 9.5: the fused softmax moves 2N elements), plus the length
    array and the argmax output when present."""
    n = rows * cols if lengths is None else int(np.clip(lengths, 0, cols).sum())
    extra = (rows * 4 if lengths is not None else 0) + (rows * 4 if argmax else 0)
    return 8 * n + extra


def sum_relu_add_bytes(rows, cols):
    return 2 * rows * cols * 4 + rows * 4


def layernorm_bytes(rows, cols):
    return 2 * rows * cols * 2 + 2 * cols * 2


def sumsq_bytes(n):
    return n * 4 + 4


def unfused_softmax_elements(M, N):
    """Element reads and writes of softmax as five separate kernels (amax,
    subtract, exp, sum, divide): reads 5MN + 2M, writes 3MN + 2M (CMU 15-779
    Lecture 8, section 3)."""
    return 5 * M * N + 2 * M, 3 * M * N + 2 * M


# ------------------------------------------------------------------ workloads


class Workload:
    """Inputs for `sets` rotating buffer sets, one launch per step, the
    logical bytes of a step and an oracle closure for the CPU baseline."""

    name = ""
    kernel = ""

    def config(self):
        raise NotImplementedError


def make_workload(name, torch, fr, synth):
    dev = "cuda"

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if name in ("softmax", "softmax_large"):
        # the headline 4096 x 1024, or the same distribution at 65536 rows
        # (256 MiB in, 256 MiB out): the largest shape of the row sweep
        rows, cols = (4096, 1024) if name == "softmax" else (65536, 1024)
        x_host = synth.softmax_inputs(rows, cols, seed=2001)
        per_set = 2 * rows * cols * 4

        class W(Workload):
            kernel = "fr_per_softmax_f32"
            bytes = softmax_bytes(rows, cols)
            dtype = "f32"

            def alloc(self, sets):
                x0 = d(x_host)
                self.x = [x0] + [x0.clone() for _ in range(sets - 1)]
                self.y = [torch.empty_like(x0) for _ in range(sets)]
                self.args = [(x, y) for x, y in zip(self.x, self.y)]

            def launch(self, k):
                x, y = self.args[k]
                fr.fr_softmax_rows(x, y)

            def output(self, k):
                return self.y[k]

            def config(self):
                p = fr.fr_plan_query(fr.FR_OP_SOFTMAX, rows, cols)
                return {"workload": f"row softmax {rows}x{cols} fp32, x ~ N(0,1)*4 with 1% entries +/-30",
                        "rows": rows, "cols": cols, "form": fr.FORM_NAMES[p.form],
                        "launch": {"threads": p.threads, "lanes_per_row": p.seg, "vec16_per_lane": p.vec,
                                   "grid": p.grid}}

            def oracle_fn(self, threads=1):
                import oracle
                if rows == 4096:
                    return (lambda: oracle.softmax_rows(x_host, threads=threads), self.bytes,
                            "full 4096x1024 batch")
                r = 4096
                return (lambda: oracle.softmax_rows(x_host[:r], threads=threads), softmax_bytes(r, cols),
                        f"first {r} of {rows} rows")

        return W(), per_set

    if name in ("sum_relu_add", "sum_relu_add_large"):
        # Example 1.1 at 64 x 128 (latency-bound), or 2^20 rows of 128
        # (1 GiB read): the largest shape of the row sweep
        rows, cols = (64, 128) if name == "sum_relu_add" else (1 << 20, 128)
        a_h, b_h, _ = synth.sum_relu_add_inputs(rows, cols, seed=1001)
        per_set = sum_relu_add_bytes(rows, cols)

        class W(Workload):
            kernel = "fr_per_sum_f32"
            bytes = sum_relu_add_bytes(rows, cols)
            dtype = "f32"

            def alloc(self, sets):
                self.args = [(d(a_h), d(b_h), torch.empty(rows, dtype=torch.float32, device=dev))
                             for _ in range(sets)]

            def launch(self, k):
                a, b, o = self.args[k]
                fr.fr_sum_relu_add(a, b, o)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                return {"workload": f"Example 1.1 sum_r 2*relu(a+b), fp32 [{rows},{cols}]"
                                    + (" (latency-bound)" if rows == 64 else ""),
                        "rows": rows, "cols": cols, "form": "per"}

            def oracle_fn(self, threads=1):
                import oracle
                if rows == 64:
                    return lambda: oracle.sum_relu_add(a_h, b_h, threads=threads), self.bytes, "full 64x128 batch"
                r = 1 << 17
                return (lambda: oracle.sum_relu_add(a_h[:r], b_h[:r], threads=threads),
                        sum_relu_add_bytes(r, cols), f"first {r} of {rows} rows")

        return W(), per_set

    if name == "c1_region":
        # 16 independent Example 1.1 sums (64 x 128 fp32): launch overhead
        # dominates ("Stax (4)", 9.9). A step is one replay of the recorded
        # region (--eager: the 16 launches one by one), timed on the host
        # loop that submits it.
        rows, cols, n = 64, 128, 16
        ins = [synth.sum_relu_add_inputs(rows, cols, seed=1001 + i)[:2] for i in range(n)]
        per_set = n * sum_relu_add_bytes(rows, cols)

        class W(Workload):
            kernel = "fr_per_sum_f32"
            bytes = n * sum_relu_add_bytes(rows, cols)
            dtype = "f32"
            host_timed = True

            def alloc(self, sets):
                self.args = [(d(a), d(b), torch.empty(rows, dtype=torch.float32, device=dev)) for a, b in ins]
                self.key = [p for t in self.args for p in (t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr())]
                self.region = fr.Region()

            def run_all(self, stream):
                for a, b, o in self.args:
                    fr.fr_sum_relu_add(a, b, o, stream=stream)

            def launch(self, k):
                if self.eager:
                    self.run_all(None)
                else:
                    self.region.run(self.key, self.run_all)

            def output(self, k):
                return self.args[-1][2]

            def config(self):
                return {"workload": "16 x Example 1.1 sum_r 2*relu(a+b), fp32 [64,128], as one recorded region"
                        if not self.eager else "16 x Example 1.1 sum_r 2*relu(a+b), fp32 [64,128], 16 launches",
                        "rows": rows, "cols": cols, "launches_per_step": n,
                        "region_state": self.region.state, "region_counts": list(self.region.counts())}

            def oracle_fn(self):
                import oracle
                return (lambda: [oracle.sum_relu_add(a, b) for a, b in ins], self.bytes,
                        f"all {n} sums")

        return W(), per_set

    if name in ("layernorm", "layernorm_large"):
        # the 2048 x 32768 workload, or the same distribution at 8192 rows
        # (512 MiB in, 512 MiB out): the largest shape measured
        rows, cols = (2048, 32768) if name == "layernorm" else (8192, 32768)
        x_h, g_h, b_h = synth.layernorm_inputs(rows, cols, seed=3001)
        per_set = 2 * rows * cols * 2

        def bf(u):
            return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).to(dev).view(torch.bfloat16)

        class W(Workload):
            kernel = "fr_per_layernorm_bf16"
            bytes = layernorm_bytes(rows, cols)
            dtype = "bf16 in/out, f32 math"

            def alloc(self, sets):
                x0 = bf(x_h)
                self.g, self.b = bf(g_h), bf(b_h)
                self.args = [(x0 if i == 0 else x0.clone(), torch.empty_like(x0)) for i in range(sets)]
                cus = torch.cuda.get_device_properties(dev).multi_processor_count
                self.plan = fr.fr_plan_query(fr.FR_OP_LAYERNORM, rows, cols, dtype=fr.FR_BF16, num_cus=cus)
                # several rows per workgroup: the pipelined kernel
                self.kernel = "fr_pipe_layernorm_bf16" if self.plan.rows_per_wg > 1 else "fr_per_layernorm_bf16"

            def launch(self, k):
                x, y = self.args[k]
                fr.fr_layernorm_rows(x, y, gamma=self.g, beta=self.b)

            def output(self, k):
                return self.args[k][1]

            def config(self):
                p = self.plan
                return {"workload": f"LayerNorm bf16 [{rows},{cols}], eps 1e-5", "rows": rows, "cols": cols,
                        "form": fr.FORM_NAMES[p.form],
                        "launch": {"threads": p.threads, "vec16_per_lane": p.vec, "rows_per_wg": p.rows_per_wg,
                                   "grid": p.grid}}

            def oracle_fn(self, threads=1):
                import oracle
                r = 128
                return (lambda: oracle.layernorm_rows(x_h[:r], g_h, b_h, threads=threads), layernorm_bytes(r, cols),
                        f"first {r} of {rows} rows")

        return W(), per_set

    if name == "sumsq":
        n = 1 << 28
        x_h = synth.sumsq_inputs(n, seed=4001)
        per_set = n * 4

        class W(Workload):
            kernel = "fr_split_sum_f32"
            bytes = sumsq_bytes(n)
            dtype = "f32"

            def alloc(self, sets):
                x0 = d(x_h)
                ws_n = fr.fr_sumsq_full_workspace_bytes(n) // 4
                self.args = [(x0 if i == 0 else x0.clone(), torch.empty(1, dtype=torch.float32, device=dev),
                              torch.empty(ws_n, dtype=torch.float32, device=dev)) for i in range(sets)]

            def launch(self, k):
                x, o, ws = self.args[k]
                fr.fr_sumsq_full(x, o, ws=ws)

            def output(self, k):
                return self.args[k][1]

            def config(self):
                return {"workload": "sum of x^2 over fp32 [2^28] to one scalar (split + finish)", "n": n,
                        "form": "split"}

            def oracle_fn(self, threads=1):
                import oracle
                m = 1 << 26
                return (lambda: oracle.sumsq(x_h[:m], threads=threads), sumsq_bytes(m),
                        "first 2^26 of 2^28 elements" + (", fixed slices per thread summed in slice order"
                                                          if threads > 1 else ""))

        return W(), per_set

    if name == "ragged":
        rows, cap = 512, 131072
        x_h, L_h = synth.ragged_softmax_inputs(rows, cap, seed=5001)
        nbytes = softmax_bytes(rows, cap, lengths=L_h, argmax=True)
        per_set = 2 * rows * cap * 4

        class W(Workload):
            kernel = "fr_split_softmax_one"
            bytes = nbytes
            dtype = "f32"

            def alloc(self, sets):
                x0 = d(x_h)
                self.L = d(L_h)
                ws_n = fr.fr_softmax_rows_workspace_bytes(rows, cap) // 4
                self.args = [(x0 if i == 0 else x0.clone(), torch.empty_like(x0),
                              torch.empty(rows, dtype=torch.int32, device=dev),
                              fr.fr_softmax_rows_workspace_init(torch.empty(ws_n, dtype=torch.float32, device=dev)))
                             for i in range(sets)]

            def launch(self, k):
                x, y, am, ws = self.args[k]
                fr.fr_softmax_rows(x, y, lengths=self.L, argmax=am, ws=ws)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                return {"workload": "ragged softmax + argmax, 512 rows padded to 131072, lengths from "
                                    "{1000,3000,50257,131071}", "rows": rows, "row_capacity": cap,
                        "valid_elements": int(L_h.sum()), "form": "split"}

            def oracle_fn(self, threads=1):
                import oracle
                r = 128
                return (lambda: oracle.softmax_rows(x_h[:r], lengths=L_h[:r], threads=threads),
                        softmax_bytes(r, cap, lengths=L_h[:r], argmax=True), f"first {r} of 512 rows")

        return W(), per_set

    if name == "copy":
        # practical ceiling and counter calibration: torch's own device copy of
        # a 4096 x 1024 fp32 buffer (16 MiB read + 16 MiB written)
        rows, cols = 4096, 1024
        per_set = 2 * rows * cols * 4

        class W(Workload):
            kernel = "copy"
            bytes = 2 * rows * cols * 4
            dtype = "f32"

            def alloc(self, sets):
                x0 = torch.randn(rows, cols, device=dev)
                self.args = [(x0 if i == 0 else x0.clone(), torch.empty_like(x0)) for i in range(sets)]

            def launch(self, k):
                x, y = self.args[k]
                y.copy_(x)

            def output(self, k):
                return self.args[k][1]

            def config(self):
                return {"workload": "plain device copy 4096x1024 fp32 (torch copy_), the practical ceiling",
                        "rows": rows, "cols": cols}

            def oracle_fn(self):
                x = np.zeros((rows, cols), dtype=np.float32)
                return lambda: x.copy(), self.bytes, "numpy copy of the same size"

        return W(), per_set

    if name in ("softmax_bwd", "softmax_bwd_large"):
        # softmax backward over the 4096 x 1024 fp32 softmax output, or the
        # same at 65536 rows (256 MiB per array)
        rows, cols = (4096, 1024) if name == "softmax_bwd" else (65536, 1024)
        x_h = synth.softmax_inputs(rows, cols, seed=2001)
        dy_h = synth.normal((rows, cols), 2001, stream=7)
        per_set = 3 * rows * cols * 4

        class W(Workload):
            kernel = "fr_per_softmax_bwd_f32"
            bytes = 3 * rows * cols * 4
            dtype = "f32"

            def alloc(self, sets):
                y0 = torch.empty((rows, cols), dtype=torch.float32, device=dev)
                fr.fr_softmax_rows(d(x_h), y0)
                g0 = d(dy_h)
                torch.cuda.synchronize()
                self.args = [(y0 if i == 0 else y0.clone(), g0 if i == 0 else g0.clone(), torch.empty_like(y0))
                             for i in range(sets)]

            def launch(self, k):
                y, g, dx = self.args[k]
                fr.fr_softmax_rows_backward(y, g, dx)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                p = fr.fr_plan_query(fr.FR_OP_SOFTMAX_BWD, rows, cols)
                return {"workload": f"softmax backward {rows}x{cols} fp32 (y = the forward output, dy ~ N(0,1))",
                        "rows": rows, "cols": cols, "form": fr.FORM_NAMES[p.form]}

            def oracle_fn(self):
                # the oracle's own forward output as its input (timing only)
                import oracle
                r = 1024
                y = oracle.softmax_rows(x_h[:r])[0].astype(np.float32)
                g = dy_h[:r].copy()
                return lambda: oracle.softmax_backward_rows(y, g), 3 * r * cols * 4, f"first {r} of {rows} rows"

        return W(), per_set

    if name == "layernorm_bwd":
        # LayerNorm backward over the 2048 x 32768 bf16 LayerNorm: dx, dgamma
        # and dbeta from the saved mean and rstd
        rows, cols = 2048, 32768
        x_h, g_h, b_h = synth.layernorm_inputs(rows, cols, seed=3001)
        dy_h = synth.to_bf16(synth.normal((rows, cols), 3001, stream=5))
        per_set = 3 * rows * cols * 2

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        class W(Workload):
            kernel = "fr_per_layernorm_bwd_bf16"
            bytes = 3 * rows * cols * 2 + cols * 2 + rows * 8 + cols * 8
            dtype = "bf16"

            def alloc(self, sets):
                x0, dy0, g = bf(x_h), bf(dy_h), bf(g_h)
                mean = torch.empty(rows, dtype=torch.float32, device=dev)
                rstd = torch.empty(rows, dtype=torch.float32, device=dev)
                fr.fr_layernorm_rows_stats(x0, torch.empty_like(x0), mean=mean, rstd=rstd, gamma=g, beta=bf(b_h))
                nbytes = fr.fr_layernorm_rows_backward_workspace_bytes(rows, cols)
                self.ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
                fr.fr_layernorm_rows_backward_workspace_init(self.ws)
                self.plan = fr.fr_plan_query(fr.FR_OP_LAYERNORM_BWD, rows, cols, dtype=fr.FR_BF16, ws_bytes=nbytes)
                self.kernel = ("fr_team_layernorm_bwd_bf16" if self.plan.form == fr.FR_FORM_SPLIT
                               else "fr_per_layernorm_bwd_bf16")
                self.g, self.mean, self.rstd = g, mean, rstd
                self.dg = torch.empty(cols, dtype=torch.float32, device=dev)
                self.db = torch.empty(cols, dtype=torch.float32, device=dev)
                self.args = [(x0 if i == 0 else x0.clone(), dy0 if i == 0 else dy0.clone(), torch.empty_like(x0))
                             for i in range(sets)]

            def launch(self, k):
                x, dy, dx = self.args[k]
                fr.fr_layernorm_rows_backward(x, dy, self.mean, self.rstd, dx, gamma=self.g, dgamma=self.dg,
                                              dbeta=self.db, ws=self.ws)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                p = self.plan
                split = p.form == fr.FR_FORM_SPLIT
                return {"workload": "LayerNorm backward 2048x32768 bf16 (dx, dgamma, dbeta from saved mean/rstd; "
                                    "dy ~ N(0,1))", "rows": rows, "cols": cols, "threads": p.threads,
                        "workgroups": p.grid, "workgroups_per_row": p.splits if split else 1,
                        "partial_rows": p.grid // p.splits if split else p.grid, "form": fr.FORM_NAMES[p.form]}

            def oracle_fn(self):
                import oracle
                r = 64
                mean, rstd = oracle.layernorm_stats(x_h[:r], eps=1e-5)
                x, dy = x_h[:r].copy(), dy_h[:r].copy()
                return (lambda: oracle.layernorm_backward_rows(x, dy, g_h, mean, rstd), 3 * r * cols * 2,
                        f"first {r} of {rows} rows")

        return W(), per_set

    if name == "add_2d":
        # x.t() + y ("Stax (4)", 9.3, Example 6.1) at 8192 x 8192 fp32: the
        # first operand transposed, staged through LDS tile by tile
        n = 8192
        x_h = synth.normal((n, n), 62, stream=1)
        y_h = synth.normal((n, n), 62, stream=2)
        per_set = 3 * n * n * 4

        class W(Workload):
            kernel = "fr_add_2d_f32"
            bytes = 3 * n * n * 4
            dtype = "f32"

            def alloc(self, sets):
                x0, y0 = d(x_h), d(y_h)
                self.args = [(x0 if i == 0 else x0.clone(), y0 if i == 0 else y0.clone(), torch.empty_like(y0))
                             for i in range(sets)]

            def launch(self, k):
                x, y, out = self.args[k]
                fr.fr_add_2d(x.t(), y, out)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                p = fr.fr_plan_query(fr.FR_OP_ADD_2D, n, n)
                return {"workload": "x.t() + y, 8192x8192 fp32 (x, y ~ N(0,1))", "rows": n, "cols": n,
                        "tile": [p.rows_per_wg, p.chunk], "form": fr.FORM_NAMES[p.form]}

            def oracle_fn(self):
                import oracle
                r = 1024
                a, b = x_h[:, :r].T, y_h[:r]
                return lambda: oracle.add_2d(a, b), 3 * r * n * 4, f"first {r} of {n} output rows"

        return W(), per_set

    if name == "gelu_bwd":
        # GELU backward ("Stax (4)", 9.3, Listing 9.3) over 2^28 fp32
        # pre-activations h ~ N(0, 4), one broadcast upstream value
        n = 1 << 28
        h_h = synth.normal((n,), 54, stream=3, std=2.0)
        per_set = 2 * n * 4

        class W(Workload):
            kernel = "fr_gelu_bwd"
            bytes = 2 * n * 4 + 4
            dtype = "f32"

            def alloc(self, sets):
                h0 = d(h_h)
                g = torch.tensor([0.5], dtype=torch.float32, device=dev)
                self.args = [(g, h0 if i == 0 else h0.clone(), torch.empty_like(h0)) for i in range(sets)]

            def launch(self, k):
                g, h, dx = self.args[k]
                fr.fr_gelu_backward(g, h, dx)

            def output(self, k):
                return self.args[k][2]

            def config(self):
                p = fr.fr_plan_query(fr.FR_OP_GELU_BWD, 1, n)
                return {"workload": "GELU backward, 2^28 fp32 (h ~ N(0,4), one broadcast dy)", "n": n,
                        "vectors_per_lane": p.vec, "grid": p.grid, "form": fr.FORM_NAMES[p.form]}

            def oracle_fn(self):
                import oracle
                m = 1 << 21
                h = h_h[:m].astype(np.float64)
                return lambda: oracle.gelu_backward(0.5, h), 8 * m, f"first {m} of {n} elements"

        return W(), per_set

    if name in ("attn_block", "attn_block_full"):
        # tiled attention ("Stax (4)", 9.10) at the pages' N = 4096, d = 128
        # (Listing 9.7: causal; attn_block_full: no mask): 4 x 16 heads bf16
        B, H, N, D = 4, 16, 4096, 128
        causal = name == "attn_block"
        q_h, k_h, v_h = synth.attn_block_inputs(B, H, H, N, N, D, seed=7001)
        per_set = 4 * B * H * N * D * 2
        pairs = N * (N + 1) // 2 if causal else N * N

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        class W(Workload):
            kernel = "fr_attn_block_bf16"
            bytes = 4 * B * H * N * D * 2 + B * H * N * 4
            flops = 4 * D * pairs * B * H
            dtype = "bf16"

            def alloc(self, sets):
                q0, k0, v0 = bf(q_h), bf(k_h), bf(v_h)
                self.args = [(q0 if i == 0 else q0.clone(), k0 if i == 0 else k0.clone(),
                              v0 if i == 0 else v0.clone(), torch.empty_like(q0),
                              torch.empty((B, H, N), dtype=torch.float32, device=dev)) for i in range(sets)]

            def launch(self, kk):
                q, k, v, o, lse = self.args[kk]
                fr.fr_attn_block(q, k, v, o, lse, causal=causal)

            def output(self, kk):
                return self.args[kk][3]

            def config(self):
                return {"workload": f"tiled attention, batch 4, 16 heads, N 4096, d 128, bf16, "
                                    f"{'causal' if causal else 'no mask'}",
                        "batch": B, "heads": H, "seq": N, "dim": D, "causal": causal, "flops_per_step": self.flops}

            def oracle_fn(self):
                import oracle
                r = 2  # query rows of one head, over all keys they see
                qf = (q_h[:1, :1, -r:].astype(np.uint32) << 16).view(np.float32)
                kf = (k_h[:1, :1].astype(np.uint32) << 16).view(np.float32)
                vf = (v_h[:1, :1].astype(np.uint32) << 16).view(np.float32)
                L = np.array([N], np.int32)
                return (lambda: [oracle.attn_decode(qf[:, :, i], kf, vf, lengths=L) for i in range(r)],
                        r * 2 * N * D * 2, f"{r} query rows of one head against all {N} keys")

        return W(), per_set

    if name == "attn_decode":
        # decode attention: batch 8, 32 query heads on 8 key-value heads,
        # 8192 keys, head dim 128, bf16 (each key and value byte read once)
        B, Hq, Hkv, S, D = 8, 32, 8, 8192, 128
        q_h, k_h, v_h, _ = synth.attn_decode_inputs(B, Hq, Hkv, S, D, seed=6001, bf16=True)
        kv_bytes = 2 * B * Hkv * S * D * 2
        nbytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4
        per_set = kv_bytes

        class W(Workload):
            kernel = "fr_attn_part"
            bytes = nbytes
            dtype = "bf16"

            def alloc(self, sets):
                bf = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
                q0, k0, v0 = bf(q_h), bf(k_h), bf(v_h)
                ws_n = fr.fr_attn_decode_workspace_bytes(B, Hq, S, D) // 4
                self.args = [(q0, k0 if i == 0 else k0.clone(), v0 if i == 0 else v0.clone(), torch.empty_like(q0),
                              torch.empty((B, Hq), dtype=torch.float32, device=dev),
                              torch.empty(ws_n, dtype=torch.float32, device=dev)) for i in range(sets)]

            def launch(self, k):
                q, kk, vv, o, lse, ws = self.args[k]
                fr.fr_attn_decode(q, kk, vv, o, lse=lse, ws=ws)

            def output(self, k):
                return self.args[k][3]

            def config(self):
                return {"workload": "decode attention, batch 8, 32 query heads on 8 key-value heads, 8192 keys, "
                                    "head dim 128, bf16", "batch": B, "heads_q": Hq, "heads_kv": Hkv, "seq": S,
                        "dim": D, "chunk_keys": 256}

            def oracle_fn(self):
                import oracle
                from_bf = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
                qs, ks, vs = from_bf(q_h[:1]), from_bf(k_h[:1]), from_bf(v_h[:1])
                return (lambda: oracle.attn_decode(qs, ks, vs), nbytes // B, "batch 1 of 8")

        return W(), per_set

    if name in ("stream_copy", "stream_copy_c3", "stream_read"):
        # practical ceilings: the library's streaming reference kernels over the
        # bytes of the softmax 4096x1024 step (16 MiB in, 16 MiB out), of the
        # LayerNorm 2048x32768 bf16 step (128 MiB in, 128 MiB out), or a
        # read-only pass over the softmax input
        nin = 16 << 20 if name != "stream_copy_c3" else 128 << 20
        reads_only = name == "stream_read"
        per_set = nin if reads_only else 2 * nin

        class W(Workload):
            kernel = "fr_stream_read_k" if reads_only else "fr_stream_copy_k"
            bytes = nin if reads_only else 2 * nin
            dtype = "u8"

            def alloc(self, sets):
                x0 = torch.randint(-2**31, 2**31 - 1, (nin // 4,), dtype=torch.int32, device=dev)
                self.args = [(x0 if i == 0 else x0.clone(),
                              torch.zeros(fr.FR_STREAM_SINK_WORDS, dtype=torch.int32, device=dev) if reads_only
                              else torch.empty_like(x0)) for i in range(sets)]

            def launch(self, k):
                x, out = self.args[k]
                if reads_only:
                    fr.fr_stream_read(x, out)
                else:
                    fr.fr_stream_copy(x, out)

            def output(self, k):
                return self.args[k][1]

            def config(self):
                what = {"stream_copy": "streaming copy of 16 MiB (the bytes of the softmax 4096x1024 step)",
                        "stream_copy_c3": "streaming copy of 128 MiB (the bytes of the LayerNorm 2048x32768 "
                                          "bf16 step)",
                        "stream_read": "streaming read of 16 MiB (the softmax 4096x1024 input)"}[name]
                return {"workload": what + ", the practical ceiling", "bytes_in": nin}

            def oracle_fn(self):
                x = np.zeros(nin // 4, dtype=np.int32)
                return lambda: x.copy(), self.bytes, "numpy copy of the same size"

        return W(), per_set

    if name == "stream_write":
        # the write half of the softmax 4096x1024 step: 16 MiB stored, nothing read
        nout = 16 << 20

        class W(Workload):
            kernel = "fr_stream_write_k"
            bytes = nout
            dtype = "u8"

            def alloc(self, sets):
                self.args = [torch.empty(nout // 4, dtype=torch.int32, device=dev) for _ in range(sets)]

            def launch(self, k):
                fr.fr_stream_write(self.args[k], 0x3F800000)

            def output(self, k):
                return self.args[k]

            def config(self):
                return {"workload": "streaming write of 16 MiB (the output of the softmax 4096x1024 step), "
                                    "the practical ceiling of the write half", "bytes_out": nout}

            def oracle_fn(self):
                return lambda: np.full(nout // 4, 1.0, dtype=np.float32), self.bytes, "numpy fill of the same size"

        return W(), nout

    if name == "empty":
        # a kernel that does nothing: back to back, the cost of one kernel
        # boundary, which every one-launch step pays whatever bytes it moves
        class W(Workload):
            kernel = "fr_empty_k"
            bytes = 0
            dtype = "none"

            def alloc(self, sets):
                # never written: the poisoned bytes are what the check expects
                self.out = torch.full((4,), -1, dtype=torch.int32, device=dev)

            def launch(self, k):
                fr.fr_stream_empty()

            def output(self, k):
                return self.out

            def config(self):
                return {"workload": "empty kernel (one workgroup), launched back to back: the floor of a "
                                    "one-launch step"}

        return W(), 1 << 30

    raise SystemExit(f"unknown workload {name}")


# ------------------------------------------------------------------ measurement


def host_facts():
    """CPU model, the host's CPU count and the CPUs this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def time_oracle(oracle_fn, budget_s):
    """GB/s of repeated oracle passes over about budget_s seconds."""
    fn, nbytes, sample = oracle_fn
    t0 = time.perf_counter()
    fn()
    one = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(one, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    dt = time.perf_counter() - t0
    return nbytes * reps / dt / 1e9, reps, dt, sample


def cpu_baseline(wl, budget_s):
    """The fp64 oracle on the host's cores: one thread, then every usable
    CPU (at most 16, the CPU share of one GPU) with rows split into
    contiguous ranges. The all-cores leg is the reported value."""
    facts = host_facts()
    one, reps1, dt1, sample = time_oracle(wl.oracle_fn(), budget_s)
    out = {"value": round(one, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{sample}, {reps1} passes in {dt1:.1f} s, single thread, fp64"}
    threads = min(16, facts["usable_cpus"])
    try:
        fn_all = wl.oracle_fn(threads=threads)
    except TypeError:
        fn_all = None  # this workload's oracle has no row-parallel leg
    if fn_all is not None and threads > 1:
        allc, reps, dt, sample = time_oracle(fn_all, budget_s)
        out = {"value": round(allc, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{sample}, {reps} passes in {dt:.1f} s, {threads} threads over row ranges, fp64",
               "one_core": {"value": round(one, 4), "cores": 1, "passes": reps1, "seconds": round(dt1, 1)}}
    out["host"] = facts
    return out


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed counter summary, if its recorded
    kernel-source digest matches the current sources; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "pointwise_reduction_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    if fields.get("csrc_sha256") != h.hexdigest() or fields.get("kernel") != kernel:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measure_latency(torch, fr):
    """lambda of Little's law ("Stax (4)", 9.1) on this device: dependent
    loads along random cycles whose entries lie 256 bytes apart (two cache
    lines), over spans that fit one XCD's L2 (4 MiB), fit the MALL (256 MB)
    but not the L2, and fit neither. L2: the cycle is walked once first and
    then measured; MALL: walked once in full, then 100k loads (12.8 MB of
    lines, three times the L2) measured; HBM: 100k loads over a 4 GiB cycle
    touched for the first time, each run on a fresh stretch of it.
    Returns one JSON-ready dict."""
    khz = fr.fr_device_clock_khz()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9001)
    stride = 256
    levels = {}
    for name, span, warm, steps in (("l2", 2 << 20, True, 20000), ("mall", 128 << 20, True, 100000),
                                    ("hbm", 4 << 30, False, 100000)):
        n = span // 4
        m = span // stride
        chain = torch.zeros(n, dtype=torch.int32, device="cuda")
        order = torch.randperm(m, generator=gen, device="cuda") * (stride // 4)
        chain[order] = torch.roll(order, -1).to(torch.int32)  # one cycle through every position
        del order
        start = 0
        if warm:
            fr.fr_pointer_chase(chain, m, start, out)  # the whole cycle once
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            fr.fr_pointer_chase(chain, steps, start, out)
            torch.cuda.synchronize()
            runs.append(int(out[0].item()) / khz * 1e6 / steps)  # ns per load
            if not warm:
                start = int(out[1].item())  # the next run continues on lines not yet touched
        levels[name] = {"span_bytes": span, "stride_bytes": stride, "loads": steps,
                        "ns_per_load": round(float(np.median(runs)), 1), "runs_ns": [round(r, 1) for r in runs]}
        del chain
        torch.cuda.empty_cache()
    lam = levels["hbm"]["ns_per_load"] * 1e-9
    q = lam * PEAK_HBM_GBS * 1e9
    return {"metric": "dependent-load latency (lambda of Little's law)", "value": levels["hbm"]["ns_per_load"],
            "unit": "ns", "n_gpus": 1, "higher_is_better": False, "levels": levels,
            "littles_law": {"peak_GBs": PEAK_HBM_GBS, "bytes_in_flight_for_peak": round(q),
                            "per_cu_bytes": round(q / 256)},
            "data": "synthetic", "config": {"workload": "pointer chase, one lane, random cycles, 256-byte spacing"}}


def run_procs(args):
    """The same measurement in args.procs child processes, one after the
    other (each its own HIP context); prints the median child's line with the
    values of all of them. This process never touches the GPU."""
    import subprocess
    argv, skip = [], False
    for a in sys.argv[1:]:
        if skip:
            skip = False
            continue
        if a == "--procs":
            skip = True
            continue
        if a.startswith("--procs="):
            continue
        argv.append(a)
    lines = []
    for i in range(args.procs):
        r = subprocess.run([sys.executable, os.path.abspath(__file__)] + argv + ["--procs", "1"] +
                           (["--no-cpu"] if i else []), capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            return r.returncode
        lines.append(json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]))
        print(f"bench.py: process {i + 1} of {args.procs}: {lines[-1]['value']} {lines[-1]['unit']}",
              file=sys.stderr, flush=True)
    vals = [ln["value"] for ln in lines]
    med = sorted(range(len(lines)), key=lambda i: vals[i])[len(lines) // 2]
    out = dict(lines[med])
    if "cpu_baseline" in lines[0]:
        out["cpu_baseline"] = lines[0]["cpu_baseline"]
    out["procs"] = {"n": len(lines), "values": vals, "median": vals[med], "min": min(vals), "max": max(vals),
                    "per_process": "median of that process's timed repetitions"}
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="softmax",
                    choices=["softmax", "softmax_large", "softmax_bwd_large", "sum_relu_add", "sum_relu_add_large",
                             "layernorm", "layernorm_large",
                             "sumsq", "ragged", "copy", "stream_copy", "stream_copy_c3", "stream_read", "stream_write", "empty", "attn_decode", "softmax_bwd", "add_2d",
                             "gelu_bwd", "layernorm_bwd", "c1_region", "attn_block",
                             "attn_block_full", "latency"])
    ap.add_argument("--warm", action="store_true", help="one buffer set: reads may hit the MALL")
    ap.add_argument("--eager", action="store_true", help="launch each step from the host (no graph)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--procs", type=int, default=3,
                    help="run the measurement in N separate processes and report the median (with the range)")
    ap.add_argument("--reps", type=int, default=3,
                    help="timed repetitions of the K steps in each process; the process reports their median")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.procs > 1:
        sys.exit(run_procs(args))

    import torch

    import pointwise_reduction_amd as fr
    import synth

    torch.cuda.set_device(0)
    dev_name = "cuda"
    if args.workload == "latency":
        print(json.dumps(measure_latency(torch, fr)), flush=True)
        return
    wl, per_set = make_workload(args.workload, torch, fr, synth)
    host_timed = getattr(wl, "host_timed", False)
    wl.eager = args.eager
    if host_timed:
        # each step is submitted by the host loop; a capturable stream (not the
        # legacy default stream) lets a recorded region record
        torch.cuda.set_stream(torch.cuda.Stream())
    sets = 1 if (args.warm or host_timed) else max(2, math.ceil(ROTATE_BYTES / per_set))
    wl.alloc(sets)
    # eager reference output of set 0
    wl.launch(0)
    torch.cuda.synchronize()
    ref_out = wl.output(0).clone()

    K, W = args.steps, args.warmup
    for k in range(W):
        wl.launch(k % sets)
    torch.cuda.synchronize()

    from pointwise_reduction_amd import timing

    # Step k of the timed region uses set k % sets. A lead-in of whole
    # rotations over the sets, in the same order, runs right before it: every
    # set is then touched once between two uses (>= 1 GiB of other buffers,
    # so no timed read is served from the 256 MB MALL, for any K), and the
    # device is busy while the timed graph is submitted.
    # The reported time comes from two device clock marks captured in the
    # same graph right before the first and right after the last timed step
    # (the lead-in runs first in that graph). Events around a replay of a
    # graph of the K steps alone, behind a lead-in replay, are reported
    # beside it: they add a fixed cost at the graph's edges.
    graph = lead = marked = mark_ms = None
    # the lead-in runs whole rotations of the buffer sets, at least LEAD_STEPS
    # steps: the device has been busy for a while (its clocks up) when the
    # first timed step starts, whatever K is
    n_lead = sets * max(1, math.ceil(LEAD_STEPS / sets))
    marks = torch.zeros(2, dtype=torch.int64, device=dev_name)
    if not (args.eager or host_timed):
        graph = timing.capture(lambda k: wl.launch(k % sets), K)
        lead = timing.capture(lambda k: wl.launch(k % sets), n_lead)
        marked = timing.capture_marked(lambda k: wl.launch(k % sets), n_lead, K,
                                       lambda i: fr.fr_device_clock(marks, i))
        clock_khz = fr.fr_device_clock_khz()
        # the marks enclose one kernel boundary more than the K steps hold
        mark_ms = timing.mark_interval(lambda k: wl.launch(k % sets), n_lead, marks,
                                       lambda i: fr.fr_device_clock(marks, i), clock_khz)
    # poison every output so the check below sees what the timed steps wrote
    for k in range(sets):
        wl.output(k).view(torch.uint8).fill_(0xFF)
    torch.cuda.synchronize()
    reps, ev_reps, raw_reps = [], [], []
    for _ in range(max(1, args.reps)):
        if graph is not None:
            raw = timing.time_marked(marked, marks, K, clock_khz) * K
            raw_reps.append(raw)
            reps.append(raw - mark_ms)
            ev_reps.append(timing.time_after_lead(lead, graph, K) * K)
        else:
            for k in range(sets if not host_timed else 0):
                wl.launch(k)
            reps.append(timing.time_eager(lambda k: wl.launch(k % sets), K) * K)
    ms = float(np.median(reps))

    # the replayed (or eager) launches computed what an eager launch computes
    same = torch.equal(wl.output(0).view(torch.uint8), ref_out.view(torch.uint8))
    if not same:
        print("bench.py: timed output differs from the eager reference", file=sys.stderr)
        sys.exit(1)

    ms_per_step = ms / K
    gbs = wl.bytes / (ms_per_step * 1e-3) / 1e9
    flops = getattr(wl, "flops", None)
    cfg = wl.config()
    timing_label = ("eager, events around the K launches" if args.eager else
                    ("host loop, one region replay per step" if host_timed else
                     "device clock marks around the K launches inside one hip graph, after a lead-in of whole "
                     "rotations over the buffer sets (>= 256 steps), less the interval of the two marks alone (their own kernel "
                     "boundary)"))
    cfg.update({"buffer_sets": sets, "rotated_bytes": sets * per_set, "timing": timing_label,
                "cache": "warm (one set)" if (args.warm or host_timed) else
                f"{sets} rotating sets, {sets * per_set / 2**30:.2f} GiB touched between two uses of a set "
                "(the 256 MB MALL cannot serve them)"})
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "reps_ms_per_step": [round(r / K, 6) for r in reps],
        "events_ms_per_step": round(float(np.median(ev_reps)) / K, 6) if ev_reps else None,
        "marks_raw_ms_per_step": round(float(np.median(raw_reps)) / K, 6) if raw_reps else None,
        "mark_interval_us": round(mark_ms * 1000, 3) if mark_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(wl.kernel, args.workload),
            "kernel": wl.kernel,
            "algorithmic_bytes_per_launch": wl.bytes,
        },
    }
    if flops:
        # a contraction: the matrix cores' dense bf16 peak bounds it
        tfs = flops / (ms_per_step * 1e-3) / 1e12
        result["value"], result["unit"] = round(tfs, 2), "TFLOP/s"
        result["roofline"].update({"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_MFMA_BF16_TFS,
                                   "unit": "TFLOP/s", "frac": round(tfs / PEAK_MFMA_BF16_TFS, 4),
                                   "algorithmic_flops_per_launch": flops, "hbm_GB_per_s": round(gbs, 2)})
    if not wl.bytes:
        # no bytes moved: the line is the time of one step
        result.update({"metric": "kernel boundary: time per step of back-to-back empty launches",
                       "value": round(ms_per_step * 1000, 4), "unit": "us", "higher_is_better": False,
                       "roofline": None})
    elif not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
