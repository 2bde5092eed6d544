"""Parity of the FP8 forward (flce_fwd_fp8) with the oracle's forward on the
dequantised inputs.

H and W are the workload's float32 draws quantised row by row to e4m3 (scale
max|row| / 448); the oracle decodes the same bytes exactly and multiplies by
the same fp32 scales, so both sides compute the loss of the same matrices.
The kernel's products are exact and accumulate in fp32, as in the bf16 path,
so the bf16 tolerances apply.
"""
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_forward_fp8
from workloads import CONFIGS, Workload, make_inputs_fp8

from gpu_helpers import TOL, rel_scalar, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WORKERS = min(16, len(os.sched_getaffinity(0)))


def _check(loss, lse, rloss, rlse, what):
    tol = TOL[torch.bfloat16]["loss"]
    e_loss = rel_scalar(loss, rloss)
    e_lse = float(np.max(np.abs(lse - rlse) / np.maximum(np.abs(rlse), 1e-30)))
    say(f"  {what}: loss rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    assert np.isfinite(loss) and np.all(np.isfinite(lse))
    assert e_loss <= tol and e_lse <= tol


CASES = [
    ((64, 128, 300), "mean"),
    ((37, 80, 1001), "sum"),        # 80 bytes per row: one partial k-stage
    ((513, 528, 2100), "mean"),     # several tiles, a k tail, ragged rows and vocabulary
    ((300, 4096, 20000), "sum"),
]


@pytest.mark.parametrize("shape,reduction", CASES)
def test_fp8_forward(shape, reduction):
    n, d, v = shape
    wl = Workload(f"fp8_{n}_{d}_{v}", n, d, v, "bf16", 0.1, "uniform", 0.1, reduction, seed=70 + n)
    hq, hs, wq, ws, y = make_inputs_fp8(wl, threads=4)
    say(f"[fp8] forward n={n} d={d} v={v} {reduction}")
    rloss, rlse = flce_forward_fp8(hq, hs, wq, ws, y, reduction=reduction)
    loss, lse = flce.linear_cross_entropy_forward_fp8(hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV),
                                                      reduction=reduction)
    torch.cuda.synchronize()
    _check(float(loss.item()), to_f64(lse), rloss, rlse, "fp8")


def test_fp8_all_rows_ignored_mean_is_zero():
    wl = Workload("fp8_ign", 40, 64, 500, "bf16", 0.1, "uniform", 0.0, "mean", seed=79)
    hq, hs, wq, ws, y = make_inputs_fp8(wl, threads=1)
    y[:] = -100
    say("[fp8] all rows ignored")
    _, rlse = flce_forward_fp8(hq, hs, wq, ws, y)
    loss, lse = flce.linear_cross_entropy_forward_fp8(hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV))
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0
    _check(0.0, to_f64(lse), 0.0, rlse, "fp8 ignored")


@pytest.mark.slow
def test_fp8_llama3_8b_head_full_size():
    wl = CONFIGS["llama3_8b_head"]
    say(f"[fp8] llama3 8b head n={wl.n} d={wl.d} v={wl.v}")
    hq, hs, wq, ws, y = make_inputs_fp8(wl)
    loss, lse = flce.linear_cross_entropy_forward_fp8(hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV),
                                                      reduction=wl.reduction)
    torch.cuda.synchronize()
    rloss, rlse = flce_forward_fp8(hq, hs, wq, ws, y, reduction=wl.reduction, workers=WORKERS)
    _check(float(loss.item()), to_f64(lse), rloss, rlse, "fp8 llama head")
