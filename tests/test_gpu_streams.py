"""Stream semantics of the C ABI: work goes on the stream it is given, and calls
on different streams may run at the same time (each has its own workspace
from the library's pool).  Every call's reduction order is fixed, so a call
made concurrently must give bitwise the results of the same call made alone."""
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from workloads import Workload, make_inputs

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(n, d, v, dtype, seed):
    wl = Workload(f"streams_{n}_{d}_{v}_{dtype}", n, d, v, dtype, 0.1, "uniform", 0.1, "mean", seed=seed)
    h, w, y = make_inputs(wl, threads=2)
    return h.to(DEV), w.to(DEV), y.to(DEV)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_streams_at_once_match_calls_alone(dtype):
    a = _inputs(300, 256, 5000, dtype, 71)
    b = _inputs(200, 128, 3001, dtype, 72)
    say(f"[streams] {dtype}: alone, then on two streams at once")
    ref_a = flce.linear_cross_entropy(*a)
    ref_b = flce.linear_cross_entropy(*b)
    ref_fa = flce.linear_cross_entropy_forward(*a)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)   # default priority
    for rep in range(3):
        with torch.cuda.stream(s1):
            out_a = flce.linear_cross_entropy(*a)
            out_fa = flce.linear_cross_entropy_forward(*a)
        with torch.cuda.stream(s2):
            out_b = flce.linear_cross_entropy(*b)
        torch.cuda.synchronize()
        for got, ref in ((out_a, ref_a), (out_b, ref_b), (out_fa, ref_fa)):
            for x, y in zip(got, ref):
                assert torch.equal(x, y), f"repeat {rep}: a concurrent call differs from the same call alone"


def test_work_is_ordered_on_the_given_stream():
    """A call on a side stream that waits for an event sees the inputs written
    before the event, and the caller's stream sees the outputs after waiting."""
    h, w, y = _inputs(256, 128, 2048, "bf16", 73)
    ref = flce.linear_cross_entropy(h, w, y)
    torch.cuda.synchronize()
    h2 = torch.zeros_like(h)
    side = torch.cuda.Stream(device=DEV)
    h2.copy_(h)                                   # on the current stream
    ev = torch.cuda.Event()
    ev.record()
    side.wait_event(ev)
    with torch.cuda.stream(side):
        out = flce.linear_cross_entropy(h2, w, y)
    torch.cuda.current_stream().wait_stream(side)
    got = [t.clone() for t in out]                # ordered after the side stream's work
    torch.cuda.synchronize()
    for x, r in zip(got, ref):
        assert torch.equal(x, r)
