"""Device timing of a launch sequence: K launches captured in a HIP graph and
replayed between two events on the launch stream.

Used by bench.py and the tuner. `launch(k)` must enqueue step k on torch's
current stream (the libfr bindings do); steps rotate over buffer sets chosen
by the caller. GPU timing of a single replay carries about 1% noise
("Stax (4)", 9.6, the remark after Proposition 9.2), so the tuner takes the
median of several replays.
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
