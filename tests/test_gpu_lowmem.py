"""flce_fwd_bwd_lowmem (forward statistics, then the backward over vocabulary
slices with the logits recomputed) against the fp64 oracle, element by element,
at sizes the oracle finishes in seconds.  Slice budgets are forced small so that
several slices (the last one ragged) and chunks inside a slice are exercised."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_forward_backward
from workloads import Workload, make_inputs

from gpu_helpers import check, say, to_f64

pytestmark = pytest.mark.gpu


def _run(h, w, y, reduction):
    hd, wd, yd = h.cuda(), w.cuda(), y.cuda()
    loss, lse, dh, dw = flce.linear_cross_entropy_lowmem(hd, wd, yd, reduction=reduction)
    torch.cuda.synchronize()
    return float(loss.item()), to_f64(lse), to_f64(dh), to_f64(dw)


# (dtype, reduction, slice budget in bytes or None for the default, chunk rows or None)
CASES = [
    ("bf16", "mean", 600_000, None),   # 768-column slices: 768, 768, 768, 196; one 300-row chunk each
    ("f32", "sum", 1_200_000, None),
    ("bf16", "sum", 600_000, "128"),   # three chunks per slice: dW's running sum inside a slice
    ("f32", "mean", 1_200_000, "128"),
    ("bf16", "mean", None, None),      # default budget: two slices of half the vocabulary
]


@pytest.mark.parametrize("dtype,reduction,budget,chunk", CASES)
def test_lowmem_parity(monkeypatch, dtype, reduction, budget, chunk):
    wl = Workload("lowmem", 300, 128, 2500, dtype, 0.1, "uniform", 0.1, reduction, seed=41)
    h, w, y = make_inputs(wl, threads=4)
    if budget is not None:
        monkeypatch.setenv("FLCE_LOWMEM_BUFFER_BYTES", str(budget))
    if chunk is not None:
        monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    p = flce.flce_lowmem_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32)
    say(f"[lowmem] {dtype} {reduction}: plan {p}")
    assert p["num_slices"] >= 2
    ref = flce_forward_backward(h, w, y, reduction=reduction)
    check(_run(h, w, y, reduction), ref, wl.torch_dtype, f"lowmem {dtype} {reduction}")


def test_lowmem_forward_matches_flce_fwd_bitwise():
    """The low-memory call's forward is the forward-only plan: loss and LSE equal flce_fwd's."""
    wl = Workload("lowmem_fwd", 300, 128, 2500, "bf16", 0.1, "uniform", 0.1, "mean", seed=42)
    h, w, y = make_inputs(wl, threads=4)
    loss, lse, _, _ = _run(h, w, y, "mean")
    lf, lsef = flce.linear_cross_entropy_forward(h.cuda(), w.cuda(), y.cuda())
    torch.cuda.synchronize()
    assert float(lf.item()) == loss and np.array_equal(to_f64(lsef), lse)


def test_lowmem_all_ignored_and_ignored_rows_zero():
    wl = Workload("lowmem_ign", 200, 128, 1500, "bf16", 0.1, "uniform", 0.3, "mean", seed=43)
    h, w, y = make_inputs(wl, threads=4)
    loss, lse, dh, dw = _run(h, w, y, "mean")
    ign = y.numpy() == -100
    assert np.all(dh[ign] == 0.0)
    check((loss, lse, dh, dw), flce_forward_backward(h, w, y), torch.bfloat16, "lowmem ignored rows")
    y_all = torch.full_like(y, -100)
    loss0, _, dh0, dw0 = _run(h, w, y_all, "mean")
    assert loss0 == 0.0 and not dh0.any() and not dw0.any()


def test_lowmem_peak_memory_llama_head():
    """At the Llama-3 head the pool's peak during the call equals the low-memory plan's
    workspace, under a fifth of the fp32 logits."""
    n, d, v = 8192, 4096, 128256
    g = torch.Generator(device="cuda").manual_seed(7)
    h = torch.randn(n, d, device="cuda", generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(v, d, device="cuda", generator=g)).to(torch.bfloat16)
    y = torch.randint(0, v, (n,), device="cuda", generator=g)
    p = flce.flce_lowmem_plan_info(n, d, v, flce.FLCE_BF16)
    torch.cuda.synchronize()
    flce.flce_memory_high_water(reset=True)
    flce.linear_cross_entropy_lowmem(h, w, y)
    torch.cuda.synchronize()
    peak = flce.flce_memory_high_water()
    say(f"[lowmem] llama head: peak {peak / 1e6:.1f} MB, plan {p['workspace_bytes'] / 1e6:.1f} MB, "
        f"fp32 logits {n * v * 4 / 1e9:.2f} GB")
    assert p["workspace_bytes"] <= peak <= p["workspace_bytes"] + (64 << 20)
    assert peak <= 0.2 * n * v * 4
