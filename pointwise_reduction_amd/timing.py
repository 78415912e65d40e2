"""Device timing of a launch sequence: K launches captured in a HIP graph and
replayed between two events on the launch stream.

Used by bench.py and the tuner. `launch(k)` must enqueue step k on torch's
current stream (the libfr bindings do); steps rotate over buffer sets chosen
by the caller. GPU timing of a single replay carries about 1% noise
("Stax (4)", 9.6, the remark after Proposition 9.2), so the tuner takes the
median of several replays.

`time_after_lead` keeps the device busy with an untimed lead-in graph while
the host submits the timed one. Events around a graph replay still carry a
fixed cost of their own at the graph's edges (about 9 us per replay on
MI355X, measured over K = 1 ... 1000 steps), which is spread over the K steps.
`capture_marked` / `time_marked` avoid it: one graph holds the lead-in, a
device clock mark, the K steps and a second mark (each mark waits, in stream
order, for the work before it). Between the marks lie the K steps and one
kernel boundary more than they contain: the one after the first mark. A
graph of the two marks alone, behind the same lead-in, measures that
boundary (`mark_interval`); subtracted, the difference is the device time
of exactly the K steps, each with the boundary to the next kernel, as in a
long run.
"""
import torch


def capture(launch, steps):
    """Capture `steps` launches into a graph; returns the graph (replayed once)."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(steps):
            launch(k)
    torch.cuda.synchronize()
    graph.replay()  # the first replay uploads the graph
    torch.cuda.synchronize()
    return graph


def time_replays(graph, steps, reps=1):
    """Milliseconds per step of each of `reps` replays."""
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / steps)
    return out


def time_after_lead(lead, graph, steps):
    """Milliseconds per step of one replay of `graph`, started right behind a
    replay of `lead` on the same stream: the start event is enqueued while
    the lead-in still runs, so it fires when the lead-in's last kernel ends
    and the timed graph's first kernel follows at once."""
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    lead.replay()
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def capture_marked(launch, lead, steps, mark):
    """One graph: `lead` untimed launches launch(0 .. lead-1), mark(0), the
    timed launches launch(0 .. steps-1), mark(1). Replayed once to upload."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(lead):
            launch(k)
        mark(0)
        for k in range(steps):
            launch(k)
        mark(1)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    return graph


def time_marked(graph, marks, steps, clock_khz, base_ms=0.0):
    """Milliseconds per step between the two clock marks of one replay of a
    capture_marked graph (marks: the int64 device tensor the marks write),
    less base_ms, the interval of the marks alone (`mark_interval`)."""
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t = marks.cpu()
    return (float(t[1] - t[0]) / clock_khz - base_ms) / steps


def mark_interval(launch, lead, marks, mark, clock_khz, reps=5):
    """Median milliseconds between two clock marks with no step between them,
    behind the same lead-in: the first mark's end and one kernel boundary."""
    graph = capture_marked(launch, lead, 0, mark)
    out = sorted(time_marked(graph, marks, 1, clock_khz) for _ in range(reps))
    del graph
    return out[len(out) // 2]


def time_eager(launch, steps):
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(steps):
        launch(k)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps
