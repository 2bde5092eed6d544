"""HIP graph capture of the library's calls.

A call enqueues only kernels and the stream-ordered allocation and release of
its workspace (no memsets, copies or host synchronisation), so a caller can
capture it into a graph and replay it.  Each test replays the graph several
times, with eager work and a synchronisation between replays, and checks every
replay against the eager result bitwise (each call's reduction order is fixed).
"""
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from workloads import Workload, make_inputs

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 5


def _inputs(dtype, seed):
    wl = Workload(f"graph_{dtype}", 300, 256, 5000, dtype, 0.1, "uniform", 0.1, "mean", seed=seed)
    return tuple(t.to(DEV) for t in make_inputs(wl, threads=2))


def _capture(fn):
    """Warm up on a side stream (as torch's capture rules ask), then capture fn()."""
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_and_check(g, outs, ref, what):
    for i in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"{what}: replay {i} differs from the eager call"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_call_in_a_graph(dtype):
    h, w, y = _inputs(dtype, 61)
    say(f"[graph] fused call, {dtype}")
    outs = (torch.empty(1, device=DEV), torch.empty(h.shape[0], device=DEV), torch.empty_like(h), torch.empty_like(w))
    flce.linear_cross_entropy(h, w, y, out=outs)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = _capture(lambda: flce.linear_cross_entropy(h, w, y, out=outs))
    _replay_and_check(g, outs, ref, f"fused {dtype}")


def test_forward_then_backward_in_a_graph():
    h, w, y = _inputs("bf16", 62)
    say("[graph] flce_fwd then flce_bwd, bf16")
    go = torch.full((1,), 0.5, device=DEV)
    dh, dw = torch.empty_like(h), torch.empty_like(w)
    state = {}

    def step():
        loss, lse = flce.linear_cross_entropy_forward(h, w, y)
        state["loss"], state["lse"] = loss, lse
        flce.linear_cross_entropy_backward(h, w, y, lse, go, out=(dh, dw))

    step()
    torch.cuda.synchronize()
    ref = [state["loss"].clone(), state["lse"].clone(), dh.clone(), dw.clone()]
    g = _capture(step)
    outs = (state["loss"], state["lse"], dh, dw)   # the graph's own forward outputs
    _replay_and_check(g, outs, ref, "forward + backward")
