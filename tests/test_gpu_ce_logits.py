"""Parity of cross-entropy on materialised logits (flce_ce_logits) with the
oracle's ce_on_logits: loss, per-row LSE and the gradient, written to a
separate buffer, over the logits in place, or from a saved LSE with an
upstream gradient; and the autograd module built on it.

Logits are drawn by the shared seeded generator (N(0, (sigma_w sqrt(d))^2),
the spread of the LM head's logits); the oracle sees the same values in
float64.  Row lengths cover the 16-byte vector path (v * sizeof(dtype) a
multiple of 16) and the element path (any other v).
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from linear_cross_entropy_bwd_amd.autograd import CrossEntropyLoss
from oracle import ce_on_logits
from workloads import Workload, make_logits

from gpu_helpers import TOL, rel_max, rel_scalar, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(n, v, dtype, ignore_frac=0.1, reduction="mean", seed=0, ignored_rows=None, sigma=None):
    wl = Workload(f"ce_{n}_{v}", n, 4096, v, dtype, 0.02, "uniform", ignore_frac, reduction,
                  ignored_rows=ignored_rows, seed=seed)
    z, y = make_logits(wl, sigma=sigma, threads=4)
    return wl, z, y


def _check(loss, lse, g, ref, dtype, what, g_up=1.0):
    tol = TOL[dtype]
    rloss, rlse, rg = ref
    e = dict(loss=rel_scalar(loss, rloss) if loss is not None else 0.0,
             lse=float(np.max(np.abs(lse - rlse) / np.maximum(np.abs(rlse), 1e-30))) if lse is not None else 0.0,
             grad=rel_max(g, g_up * rg) if g is not None else 0.0)
    say(f"  {what} errors {e}")
    if loss is not None:
        assert np.isfinite(loss) and e["loss"] <= tol["loss"], f"{what} loss {loss} vs {rloss}"
    if lse is not None:
        assert np.all(np.isfinite(lse)) and e["lse"] <= tol["loss"], f"{what} lse"
    if g is not None:
        assert np.all(np.isfinite(g)) and e["grad"] <= tol["grad"], f"{what} grad"


# Rows of 16-byte vectors run register-resident (256 threads up to 64 KB rows,
# 1024 threads up to 256 KB), longer rows and other lengths stream twice.
CASES = [
    ((64, 300), "f32", "mean"),       # 1200-byte rows: resident, 256 threads x 1 vector
    ((37, 301), "f32", "sum"),        # element path
    ((37, 1001), "bf16", "mean"),     # element path, ragged
    ((129, 4096), "bf16", "mean"),    # resident, 256 x 2
    ((300, 32000), "bf16", "sum"),    # resident, 256 x 16
    ((65, 5003), "f32", "mean"),      # element path
    ((33, 50000), "bf16", "mean"),    # resident, 1024 x 8, the later threads hold fewer vectors
    ((19, 40000), "f32", "sum"),      # resident, 1024 x 16
    ((17, 151936), "bf16", "mean"),   # 297 KB rows: streamed twice, 16-byte vectors
    ((9, 70000), "f32", "mean"),      # 280 KB rows: streamed twice
]


@pytest.mark.parametrize("shape,dtype,reduction", CASES)
@pytest.mark.parametrize("grad", [None, "separate", "inplace"])
def test_ce_forward_and_gradient(shape, dtype, reduction, grad):
    n, v = shape
    wl, z, y = _case(n, v, dtype, reduction=reduction, seed=40 + n)
    say(f"[ce] n={n} v={v} {dtype} {reduction} grad={grad}")
    ref = ce_on_logits(z, y, reduction=reduction)
    zd, yd = z.to(DEV), y.to(DEV)
    loss, lse, g = flce.cross_entropy(zd, yd, reduction=reduction, grad=grad)
    torch.cuda.synchronize()
    if grad == "inplace":
        assert g.data_ptr() == zd.data_ptr()
    else:
        assert torch.equal(zd.cpu(), z), "logits were modified"
    _check(float(loss.item()), to_f64(lse), None if g is None else to_f64(g), ref, wl.torch_dtype, "ce")


@pytest.mark.parametrize("shape,dtype", [((64, 300), "f32"), ((37, 1001), "bf16"), ((129, 4096), "bf16")])
@pytest.mark.parametrize("inplace", [False, True])
def test_ce_backward_from_saved_lse(shape, dtype, inplace):
    n, v = shape
    wl, z, y = _case(n, v, dtype, seed=50 + n)
    say(f"[ce] backward from lse n={n} v={v} {dtype} inplace={inplace}")
    rloss, rlse, rg = ce_on_logits(z, y)
    zd, yd = z.to(DEV), y.to(DEV)
    lse = torch.from_numpy(rlse.astype(np.float32)).to(DEV)
    g_up = -1.5
    go = torch.tensor([g_up], dtype=torch.float32, device=DEV)
    g = flce.cross_entropy_backward(zd, yd, lse, go, out=zd if inplace else None)
    torch.cuda.synchronize()
    _check(None, None, to_f64(g), (rloss, rlse, rg), wl.torch_dtype, "ce bwd", g_up=g_up)


def test_ce_ignored_rows_and_empty_mean():
    wl, z, y = _case(96, 1000, "f32", ignore_frac=0.0, ignored_rows=(10, 40), seed=3)
    say("[ce] ignored block")
    ref = ce_on_logits(z, y)
    loss, lse, g = flce.cross_entropy(z.to(DEV), y.to(DEV), grad="separate")
    torch.cuda.synchronize()
    gh = to_f64(g)
    assert np.all(gh[10:40] == 0.0)
    _check(float(loss.item()), to_f64(lse), gh, ref, wl.torch_dtype, "ce ignored")
    # every row ignored: mean loss and gradient are 0, the LSE is still returned
    y_all = torch.full_like(y, -100)
    loss, lse, g = flce.cross_entropy(z.to(DEV), y_all.to(DEV), grad="separate")
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0 and not torch.any(g != 0)
    _check(None, to_f64(lse), None, ref, wl.torch_dtype, "ce all ignored lse")


def test_ce_extreme_logits_stay_finite():
    # A logit far above the rest: the online max keeps every exp in range.
    wl, z, y = _case(16, 4096, "f32", ignore_frac=0.0, seed=9)
    z[:, 7] = 1.0e4
    z[3, :] = -3.0e4
    say("[ce] extreme logits")
    ref = ce_on_logits(z, y)
    loss, lse, g = flce.cross_entropy(z.to(DEV), y.to(DEV), grad="separate")
    torch.cuda.synchronize()
    _check(float(loss.item()), to_f64(lse), to_f64(g), ref, wl.torch_dtype, "ce extreme")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ce_autograd_module(dtype):
    wl, z, y = _case(48, 2048, dtype, seed=11)
    say(f"[ce] autograd {dtype}")
    rloss, rlse, rg = ce_on_logits(z, y, reduction="sum")
    zd = z.to(DEV).requires_grad_(True)
    loss = CrossEntropyLoss(reduction="sum")(zd, y.to(DEV))
    (loss * 0.5).backward()
    torch.cuda.synchronize()
    _check(float(loss.item()), None, to_f64(zd.grad), (rloss, rlse, rg), wl.torch_dtype, "ce autograd", g_up=0.5)


def test_ce_llama3_8b_head_logits_sampled():
    # Logits of the Llama-3 8B head at its bench size: 8192 x 128256 bf16
    # (about 2.1 GB), gradient in place; the oracle checks sampled rows and
    # the loss is checked against the oracle over every row.
    n, v = 8192, 128256
    wl, z, y = _case(n, v, "bf16", ignore_frac=0.05, seed=2)
    say(f"[ce] llama3 8b head logits n={n} v={v}")
    zd, yd = z.to(DEV), y.to(DEV)
    loss, lse, g = flce.cross_entropy(zd, yd, grad="inplace")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(5).integers(0, n, 29)]))
    _, rlse_s, rg_s = ce_on_logits(z[rows], y[rows], reduction="sum")
    nvalid = int((y != -100).sum())
    lse_h = to_f64(lse)
    rloss_all = _loss_all_rows(z, y, nvalid)
    _check(float(loss.item()), lse_h[rows], to_f64(g[rows]) * nvalid, (rloss_all, rlse_s, rg_s), wl.torch_dtype,
           "ce llama head")


def _loss_all_rows(z, y, nvalid):
    # mean loss over every row from the oracle, a block of rows at a time
    total = 0.0
    for lo in range(0, z.shape[0], 512):
        l, _, _ = ce_on_logits(z[lo:lo + 512], y[lo:lo + 512], reduction="sum")
        total += l
    return total / nvalid


def test_ce_more_rows_than_one_grid():
    # 65537 rows: the row kernels' grid stops at 65536 workgroups and loops for the rest.
    wl, z, y = _case(65537, 64, "bf16", seed=13)
    say("[ce] 65537 rows")
    ref = ce_on_logits(z, y)
    loss, lse, g = flce.cross_entropy(z.to(DEV), y.to(DEV), grad="separate")
    torch.cuda.synchronize()
    _check(float(loss.item()), to_f64(lse), to_f64(g), ref, wl.torch_dtype, "ce 65537 rows")
    loss_f, lse_f, _ = flce.cross_entropy(z.to(DEV), y.to(DEV), grad=None)
    torch.cuda.synchronize()
    _check(float(loss_f.item()), to_f64(lse_f), None, ref, wl.torch_dtype, "ce 65537 rows, forward")


def test_wrappers_check_saved_lse_scale_and_outputs():
    """A misshaped or wrongly typed saved LSE, upstream scale or output buffer raises
    ValueError in the wrappers, before the library is called."""
    n, v = 16, 300
    z = torch.randn(n, v, device=DEV, dtype=torch.bfloat16)
    y = torch.randint(0, v, (n,), device=DEV)
    lse = torch.zeros(n, dtype=torch.float32, device=DEV)
    for bad_lse in (lse[:-1], lse.double(), torch.zeros(2 * n, device=DEV)[::2]):
        with pytest.raises(ValueError):
            flce.cross_entropy_backward(z, y, bad_lse)
    with pytest.raises(ValueError):
        flce.cross_entropy_backward(z, y, lse, torch.ones(2, device=DEV))
    with pytest.raises(ValueError):
        flce.cross_entropy_backward(z, y, lse, out=torch.empty(n, v, device=DEV))      # fp32 for bf16 logits
    g = flce.cross_entropy_backward(z.clone(), y, lse, out=None)
    assert g.shape == z.shape
    h = torch.randn(n, 64, device=DEV, dtype=torch.bfloat16)
    w = torch.randn(v, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_backward(h, w, y, lse[:-1])
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_backward(h, w, y, lse, out=(torch.empty_like(h), torch.empty(v, 32, device=DEV,
                                                                                                dtype=torch.bfloat16)))
    with pytest.raises(ValueError):
        flce.linear_cross_entropy(h, w, y, out=(torch.empty(1, device=DEV), torch.empty(n, device=DEV),
                                                torch.empty_like(h), torch.empty_like(w).t()))
