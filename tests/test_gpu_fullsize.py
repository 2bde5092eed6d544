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


# The oracle's fp64 forward of each workload, computed once per test session.
_FWD = {}


def _oracle_forward(wl, h, w64, y):
    if wl.name not in _FWD:
        _FWD[wl.name] = flce_forward(h, w64, y, reduction=wl.reduction, workers=WORKERS)
    return _FWD[wl.name]


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
    rloss, rlse = _oracle_forward(wl, h, w64, y)
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


def _check_gradients_sampled(wl, h, w64, y, rlse, dh, dw, chunk, what):
    dev = dh.device
    tol = TOL[torch.bfloat16]
    yn = y.numpy()
    rng = np.random.default_rng(4343)
    rows = _sample_rows(wl.n, chunk, yn, rng)
    _, rdh = flce_rows(h, w64, y, rows, reduction=wl.reduction)
    e_dh = rel_max(to_f64(dh[torch.as_tensor(rows, device=dev)]), rdh)
    cols = _sample_vocab(wl.v, yn, rng)
    rdw = flce_dw_rows(h, w64, y, rlse, cols, reduction=wl.reduction)
    e_dw = rel_max(to_f64(dw[torch.as_tensor(cols, device=dev)]), rdw)
    say(f"  {what}: sampled dH rows {len(rows)}: {e_dh:.2e}; sampled dW rows {len(cols)}: {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]


@pytest.mark.parametrize("name", ["llama3_8b_head", "qwen2_head", "long_context", "stability_stress"])
def test_full_size_forward_only(name):
    """flce_fwd alone at full size: the loss and every row's LSE against the oracle's forward."""
    wl = CONFIGS[name]
    h, w, y = make_inputs(wl)
    loss, lse = flce.linear_cross_entropy_forward(h.cuda(), w.cuda(), y.cuda(), reduction=wl.reduction)
    torch.cuda.synchronize()
    rloss, rlse = _oracle_forward(wl, h, to_f64(w), y)
    e_loss = rel_scalar(float(loss.item()), rloss)
    e_lse = float(np.max(np.abs(to_f64(lse) - rlse) / np.abs(rlse)))
    say(f"[fullsize fwd] {name}: loss rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    tol = TOL[torch.bfloat16]
    assert e_loss <= tol["loss"] and e_lse <= tol["loss"]


@pytest.mark.parametrize("name", ["llama3_8b_head", "qwen2_head"])
def test_full_size_lowmem(name):
    """flce_fwd_bwd_lowmem at full size: loss and LSE against the oracle's forward, sampled
    dH and dW rows, ignored rows' zero dH, and the workspace against the fp32 logits."""
    wl = CONFIGS[name]
    h, w, y = make_inputs(wl)
    p = flce.flce_lowmem_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16)
    say(f"[fullsize lowmem] {name}: plan {p}")
    hd, wd, yd = h.cuda(), w.cuda(), y.cuda()
    torch.cuda.synchronize()
    flce.flce_memory_high_water(reset=True)
    loss, lse, dh, dw = flce.linear_cross_entropy_lowmem(hd, wd, yd, reduction=wl.reduction)
    torch.cuda.synchronize()
    peak = flce.flce_memory_high_water()
    say(f"  peak {peak / 1e6:.1f} MB = {peak / (wl.n * wl.v * 4):.3f} of the fp32 logits")
    assert peak < 0.2 * wl.n * wl.v * 4 or name != "llama3_8b_head"
    ign = torch.from_numpy(y.numpy() == -100).to(dh.device)
    assert bool((dh[ign] == 0).all())
    w64 = to_f64(w)
    rloss, rlse = _oracle_forward(wl, h, w64, y)
    e_loss = rel_scalar(float(loss.item()), rloss)
    e_lse = float(np.max(np.abs(to_f64(lse) - rlse) / np.abs(rlse)))
    say(f"  loss rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    tol = TOL[torch.bfloat16]
    assert e_loss <= tol["loss"] and e_lse <= tol["loss"]
    _check_gradients_sampled(wl, h, w64, y, rlse, dh, dw, wl.n, "lowmem")


def test_stress_all_ignored_chunk(monkeypatch):
    """The stability-stress workload with 4096-row chunks, so that its ignored block
    [4096, 8192) is exactly one whole chunk between valid chunks: that chunk adds
    nothing to dW, its dH rows are zero, and the result matches the oracle."""
    wl = CONFIGS["stability_stress"]
    monkeypatch.setenv("FLCE_CHUNK_ROWS", "4096")
    plan = flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16, 1)
    assert plan["chunk_rows"] == 4096 and plan["num_chunks"] == 4
    h, w, y = make_inputs(wl)
    yn = y.numpy()
    assert np.all(yn[4096:8192] == -100) and np.all(yn[:4096] != -100) and np.all(yn[8192:] != -100)
    loss, lse, dh, dw = flce.linear_cross_entropy(h.cuda(), w.cuda(), y.cuda(), reduction=wl.reduction)
    torch.cuda.synchronize()
    assert bool((dh[4096:8192] == 0).all())
    w64 = to_f64(w)
    rloss, rlse = _oracle_forward(wl, h, w64, y)
    e_loss = rel_scalar(float(loss.item()), rloss)
    e_lse = float(np.max(np.abs(to_f64(lse) - rlse) / np.abs(rlse)))
    say(f"[stress, ignored chunk] loss rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    assert e_loss <= TOL[torch.bfloat16]["loss"] and e_lse <= TOL[torch.bfloat16]["loss"]
    _check_gradients_sampled(wl, h, w64, y, rlse, dh, dw, 4096, "ignored chunk")


@pytest.mark.parametrize("name", ["llama3_8b_head", "stability_stress"])
def test_full_size_gradient_forms_agree(monkeypatch, name):
    """The per-row factor form (default) against the in-place form of the gradient
    (FLCE_INPLACE_GRAD=1) at full size: the forward is shared, so loss and every
    LSE are bitwise equal; dH and dW agree to within the bf16 gradient tolerance on
    every element.  The stability-stress workload flags nearly every row."""
    wl = CONFIGS[name]
    say(f"[fullsize] gradient forms, {name}")
    h, w, y = make_inputs(wl)
    dev = torch.device("cuda:0")
    hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
    assert flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16, 1)["folded_factor"] == 1
    loss_f, lse_f, dh_f, dw_f = flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction)
    monkeypatch.setenv("FLCE_INPLACE_GRAD", "1")
    assert flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16, 1)["folded_factor"] == 0
    loss_i, lse_i, dh_i, dw_i = flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction)
    torch.cuda.synchronize()
    assert torch.equal(loss_f, loss_i) and torch.equal(lse_f, lse_i)
    tol = TOL[torch.bfloat16]["grad"]
    for a, b, what in ((dh_f, dh_i, "dH"), (dw_f, dw_i, "dW")):
        err = float((a.float() - b.float()).abs().max()) / float(b.float().abs().max())
        say(f"  {what}: max|folded - in place| / max|in place| = {err:.2e}")
        assert err <= tol, what
    del hd, wd, yd, dh_f, dw_f, dh_i, dw_i
    torch.cuda.empty_cache()
