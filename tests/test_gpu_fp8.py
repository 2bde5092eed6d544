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


# --- backward from the saved LSE --------------------------------------------------

def _deq(q, s):
    from oracle import decode_e4m3
    return decode_e4m3(q.numpy()) * s.double().numpy()[:, None]


@pytest.mark.parametrize("shape,reduction", CASES[:3])
def test_fp8_backward_from_oracle_lse(shape, reduction):
    """flce_bwd_fp8 from the oracle's LSE (rounded to fp32), upstream gradient 0.5: dH
    and dW against the oracle's backward on the dequantised matrices (the kernels
    round the dequantised H and W to bf16 for the two contractions)."""
    from oracle import flce_backward_fp8
    n, d, v = shape
    wl = Workload(f"fp8b_{n}_{d}_{v}", n, d, v, "bf16", 0.1, "uniform", 0.1, reduction, seed=80 + n)
    hq, hs, wq, ws, y = make_inputs_fp8(wl, threads=4)
    say(f"[fp8] backward n={n} d={d} v={v} {reduction}")
    _, rlse = flce_forward_fp8(hq, hs, wq, ws, y, reduction=reduction)
    lse32 = rlse.astype(np.float32)
    rdh, rdw = flce_backward_fp8(hq, hs, wq, ws, y, lse32.astype(np.float64), grad_out=0.5, reduction=reduction)
    go = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    dh, dw = flce.linear_cross_entropy_backward_fp8(hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV),
                                                    torch.from_numpy(lse32).to(DEV), go, reduction=reduction)
    torch.cuda.synchronize()
    from gpu_helpers import rel_max
    e = dict(dh=rel_max(to_f64(dh), rdh), dw=rel_max(to_f64(dw), rdw))
    say(f"  errors {e}")
    tol = TOL[torch.bfloat16]["grad"]
    assert e["dh"] <= tol and e["dw"] <= tol


def test_fp8_forward_then_backward_end_to_end():
    from oracle import flce_forward_backward
    from gpu_helpers import rel_max
    n, d, v = 300, 256, 5000
    wl = Workload("fp8_e2e", n, d, v, "bf16", 0.1, "uniform", 0.1, "mean", seed=85)
    hq, hs, wq, ws, y = make_inputs_fp8(wl, threads=4)
    say("[fp8] forward then backward, end to end")
    _, _, rdh, rdw = flce_forward_backward(_deq(hq, hs), _deq(wq, ws), y)
    args = (hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV))
    _, lse = flce.linear_cross_entropy_forward_fp8(*args)
    dh, dw = flce.linear_cross_entropy_backward_fp8(*args, lse)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]["grad"]
    assert rel_max(to_f64(dh), rdh) <= tol and rel_max(to_f64(dw), rdw) <= tol


@pytest.mark.slow
def test_fp8_backward_llama3_8b_head_full_size():
    from oracle import flce_dw_rows, flce_rows
    from gpu_helpers import rel_max
    wl = CONFIGS["llama3_8b_head"]
    say(f"[fp8] backward llama3 8b head n={wl.n} d={wl.d} v={wl.v}")
    hq, hs, wq, ws, y = make_inputs_fp8(wl)
    h64, w64 = _deq(hq, hs), _deq(wq, ws)
    _, rlse = flce_forward_fp8(hq, hs, wq, ws, y, reduction=wl.reduction, workers=WORKERS)
    lse32 = rlse.astype(np.float32)
    dh, dw = flce.linear_cross_entropy_backward_fp8(hq.to(DEV), hs.to(DEV), wq.to(DEV), ws.to(DEV), y.to(DEV),
                                                    torch.from_numpy(lse32).to(DEV), reduction=wl.reduction)
    torch.cuda.synchronize()
    rng = np.random.default_rng(93)
    rows = sorted({0, wl.n - 1, *(int(r) for r in rng.choice(wl.n, 12, replace=False))})
    _, rdh = flce_rows(h64, w64, y, rows, reduction=wl.reduction)
    cols = sorted({0, wl.v - 1, *(int(c) for c in rng.choice(wl.v, 8, replace=False))})
    rdw = flce_dw_rows(h64, w64, y, lse32.astype(np.float64), cols, reduction=wl.reduction)
    e_dh = rel_max(to_f64(dh[torch.tensor(rows, device=DEV)]), rdh)
    e_dw = rel_max(to_f64(dw[torch.tensor(cols, device=DEV)]), rdw)
    say(f"  sampled dH rel {e_dh:.2e}, dW rel {e_dw:.2e}")
    tol = TOL[torch.bfloat16]["grad"]
    assert e_dh <= tol and e_dw <= tol


def test_fp8_wrappers_check_inputs():
    """Wrong label dtype, non-contiguous codes, short scales and a misshaped LSE raise
    ValueError in the wrappers, before the library is called."""
    wl = Workload("fp8_checks", 8, 32, 64, "bf16", 0.1, "uniform", 0.0, "mean", seed=90)
    hq, hs, wq, ws, y = (t.to(DEV) for t in make_inputs_fp8(wl, threads=1))
    lse = torch.zeros(8, dtype=torch.float32, device=DEV)
    bad = [
        (hq, hs, wq, ws, y.to(torch.int32)),
        (hq.t().contiguous().t(), hs, wq, ws, y),
        (hq, hs[:-1], wq, ws, y),
        (hq, hs, wq, ws[:-1], y),
    ]
    for args in bad:
        with pytest.raises(ValueError):
            flce.linear_cross_entropy_forward_fp8(*args)
        with pytest.raises(ValueError):
            flce.linear_cross_entropy_backward_fp8(*args, lse)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_backward_fp8(hq, hs, wq, ws, y, lse[:-1])
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_backward_fp8(hq, hs, wq, ws, y, lse, torch.ones(2, device=DEV))
