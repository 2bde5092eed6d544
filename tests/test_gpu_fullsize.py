"""Parity at the full benchmark sizes, in the launch configuration bench.py times.

The oracle evaluates the whole forward in fp64 (loss and every row's LSE),
dH on sampled token rows and dW on sampled vocabulary rows (using its own
LSE), and the GPU result must match at the bf16 tolerances.  Properties that
hold at any size are checked on every element: ignored rows have a zero dH
row, and the dW rows sum to zero up to the output rounding.
"""
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_dw_rows, flce_forward, flce_rows
from workloads import CONFIGS, make_inputs

from gpu_helpers import TOL, rel_max, rel_scalar, say, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WORKERS = min(16, len(os.sched_getaffinity(0)))


def _sample_rows(n, chunk, y, rng):
    rows = {0, n - 1}
    for c in range(chunk, n, chunk):
        rows.update({c - 1, c})
    rows.update(int(r) for r in rng.choice(n, size=16, replace=False))
    ign = np.flatnonzero(y == -100)
    if ign.size:
        rows.update(int(r) for r in rng.choice(ign, size=min(4, ign.size), replace=False))
    return sorted(r for r in rows if 0 <= r < n)


def _sample_vocab(v, y, rng):
    cols = {0, 1, v - 1, v - 2}
    valid = y[y >= 0]
    cols.update(int(c) for c in rng.choice(valid, size=6, replace=False))     # some label ids
    cols.update(int(c) for c in rng.choice(v, size=6, replace=False))
    return sorted(cols)


@pytest.mark.parametrize("name", ["llama3_8b_head", "qwen2_head", "long_context", "stability_stress"])
def test_full_size(name):
    wl = CONFIGS[name]
    say(f"[fullsize] {name}: n={wl.n} d={wl.d} v={wl.v} {wl.dtype} {wl.reduction}")
    h, w, y = make_inputs(wl)
    dev = torch.device("cuda:0")
    hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
    plan = flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16, 1)
    say(f"  plan {plan}")
    loss, lse, dh, dw = flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction)
    torch.cuda.synchronize()
    loss = float(loss.item())
    lse = to_f64(lse)
    yn = y.numpy()
    ign = yn == -100
    say(f"  gpu loss {loss:.6f}")
    tol = TOL[torch.bfloat16]

    # properties on every element
    dh_ign = dh[torch.from_numpy(ign).to(dev)] if ign.any() else None
    if dh_ign is not None:
        assert bool((dh_ign == 0).all()), "ignored rows must have a zero dH row"
    colsum = dw.float().sum(dim=0).double()
    abssum = dw.float().abs().sum(dim=0).double()
    assert bool((colsum.abs() <= abssum * 2.0 ** -8 + 1e-30).all()), "dW rows must sum to zero"
    assert bool(torch.isfinite(dh).all()) and bool(torch.isfinite(dw).all())

    # oracle: whole forward in fp64
    w64 = to_f64(w)
    rloss, rlse = flce_forward(h, w64, y, reduction=wl.reduction, workers=WORKERS)
    e_loss = rel_scalar(loss, rloss)
    e_lse = float(np.max(np.abs(lse - rlse) / np.abs(rlse)))
    say(f"  oracle loss {rloss:.6f}: rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    assert e_loss <= tol["loss"] and e_lse <= tol["loss"]

    rng = np.random.default_rng(4242)
    rows = _sample_rows(wl.n, plan["chunk_rows"], yn, rng)
    _, rdh = flce_rows(h, w64, y, rows, reduction=wl.reduction)
    gdh = to_f64(dh[torch.as_tensor(rows, device=dev)])
    e_dh = rel_max(gdh, rdh)
    cols = _sample_vocab(wl.v, yn, rng)
    rdw = flce_dw_rows(h, w64, y, rlse, cols, reduction=wl.reduction)
    gdw = to_f64(dw[torch.as_tensor(cols, device=dev)])
    e_dw = rel_max(gdw, rdw)
    say(f"  sampled dH rows {len(rows)}: {e_dh:.2e}; sampled dW rows {len(cols)}: {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]
