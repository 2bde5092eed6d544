"""Shared helpers of the GPU parity tests: run the library through its C ABI
and compare with the oracle at the fp32 / bf16 tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_cross_entropy_bwd_amd as flce

# Tolerances: relative error of the loss (and of each LSE element) and
# max|err| / max|ref| for dH and dW.
TOL = {
    torch.float32: dict(loss=1e-5, grad=1e-4),
    torch.bfloat16: dict(loss=2e-3, grad=2e-2),
}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_f64(t) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.double().numpy()


def run_lib(h, w, y, reduction="mean", ignore_index=-100, dev="cuda:0"):
    """Inputs are CPU tensors; returns (loss, lse, dh, dw) as float64 numpy."""
    hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
    loss, lse, dh, dw = flce.linear_cross_entropy(hd, wd, yd, ignore_index=ignore_index, reduction=reduction)
    torch.cuda.synchronize()
    return float(loss.item()), to_f64(lse), to_f64(dh), to_f64(dw)


def rel_max(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    return err / den if den > 0 else err


def rel_scalar(a, b) -> float:
    return abs(a - b) / abs(b) if b != 0 else abs(a - b)


def check(gpu, ref, dtype, what=""):
    """Assert the loss, LSE, dH and dW tolerances; return the measured errors."""
    tol = TOL[dtype]
    loss, lse, dh, dw = gpu
    rloss, rlse, rdh, rdw = ref
    e = dict(
        loss=rel_scalar(loss, rloss),
        lse=float(np.max(np.abs(lse - rlse) / np.maximum(np.abs(rlse), 1e-30))) if lse.size else 0.0,
        dh=rel_max(dh, rdh),
        dw=rel_max(dw, rdw),
    )
    say(f"  {what} errors {e}")
    assert np.isfinite(loss) and np.all(np.isfinite(lse)) and np.all(np.isfinite(dh)) and np.all(np.isfinite(dw))
    assert e["loss"] <= tol["loss"], f"{what} loss {loss} vs {rloss}"
    assert e["lse"] <= tol["loss"], f"{what} lse"
    assert e["dh"] <= tol["grad"], f"{what} dH"
    assert e["dw"] <= tol["grad"], f"{what} dW"
    return e
