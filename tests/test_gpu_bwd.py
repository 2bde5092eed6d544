"""Parity of the backward from the saved LSE (flce_bwd, recompute) and of its
autograd wrapper.

The saved LSE fed to flce_bwd comes from the oracle (fp64, rounded to fp32),
so the expected gradients are the oracle's backward from that same LSE.  The
end-to-end tests run the library's forward and then its backward and compare
with the oracle's forward-backward gradients times the upstream gradient.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from linear_cross_entropy_bwd_amd.autograd import LinearCrossEntropyLoss
from oracle import flce_backward_from_lse, flce_forward, flce_forward_backward
from workloads import Workload, make_inputs

from gpu_helpers import TOL, rel_max, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(n, d, v, dtype, sigma_w=0.1, ignore_frac=0.1, reduction="mean", seed=0):
    wl = Workload(f"bwd_{n}_{d}_{v}", n, d, v, dtype, sigma_w, "uniform", ignore_frac, reduction, seed=seed)
    return wl, make_inputs(wl, threads=4)


def _check_grads(dh, dw, rdh, rdw, dtype, what):
    tol = TOL[dtype]["grad"]
    e = dict(dh=rel_max(dh, rdh), dw=rel_max(dw, rdw))
    say(f"  {what} errors {e}")
    assert np.all(np.isfinite(dh)) and np.all(np.isfinite(dw))
    assert e["dh"] <= tol, f"{what} dH"
    assert e["dw"] <= tol, f"{what} dW"


CASES = [
    ((64, 72, 300), "f32", "mean"),
    ((37, 72, 1001), "bf16", "mean"),
    ((37, 72, 1001), "f32", "sum"),
    ((513, 520, 2100), "bf16", "mean"),
    ((300, 256, 20000), "bf16", "sum"),     # dH splits its vocabulary reduction
]


@pytest.mark.parametrize("shape,dtype,reduction", CASES)
def test_bwd_from_oracle_lse(shape, dtype, reduction):
    n, d, v = shape
    wl, (h, w, y) = _case(n, d, v, dtype, reduction=reduction, seed=30 + n)
    say(f"[bwd] from oracle lse: n={n} d={d} v={v} {dtype} {reduction}")
    _, lse64 = flce_forward(h, w, y, reduction=reduction)
    lse32 = torch.from_numpy(lse64.astype(np.float32))
    g_up = 0.75
    rdh, rdw = flce_backward_from_lse(h, w, y, lse32.double().numpy(), grad_out=g_up, reduction=reduction)
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    go = torch.tensor([g_up], dtype=torch.float32, device=DEV)
    dh, dw = flce.linear_cross_entropy_backward(hd, wd, yd, lse32.to(DEV), go, reduction=reduction)
    torch.cuda.synchronize()
    _check_grads(to_f64(dh), to_f64(dw), rdh, rdw, wl.torch_dtype, "bwd")


@pytest.mark.parametrize("chunk,chunks,paired", [("128", 3, 0), ("80", 4, 1), ("64", 5, 1), ("512", 1, 0)])
def test_bwd_chunk_modes_bf16(monkeypatch, chunk, chunks, paired):
    """Interior 256x256 tiles with first/middle/last and single-chunk dW accumulation,
    chunk by chunk and over chunk pairs."""
    wl, (h, w, y) = _case(300, 256, 1500, "bf16", seed=33)
    monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    p = flce.flce_plan_info(300, 256, 1500, flce.FLCE_BF16, 1)
    assert (p["num_chunks"], p["dw_pairs"]) == (chunks, paired)
    _, lse64 = flce_forward(h, w, y)
    lse32 = torch.from_numpy(lse64.astype(np.float32))
    rdh, rdw = flce_backward_from_lse(h, w, y, lse32.double().numpy())
    dh, dw = flce.linear_cross_entropy_backward(h.to(DEV), w.to(DEV), y.to(DEV), lse32.to(DEV))
    torch.cuda.synchronize()
    _check_grads(to_f64(dh), to_f64(dw), rdh, rdw, torch.bfloat16, f"bwd chunk {chunk}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_then_backward_end_to_end(dtype):
    wl, (h, w, y) = _case(200, 136, 3000, dtype, seed=34)
    _, _, rdh, rdw = flce_forward_backward(h, w, y)
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    _, lse = flce.linear_cross_entropy_forward(hd, wd, yd)
    go = torch.tensor([-1.5], dtype=torch.float32, device=DEV)
    dh, dw = flce.linear_cross_entropy_backward(hd, wd, yd, lse, go)
    torch.cuda.synchronize()
    _check_grads(to_f64(dh), to_f64(dw), -1.5 * rdh, -1.5 * rdw, wl.torch_dtype, "fwd+bwd")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_module(dtype):
    wl, (h, w, y) = _case(150, 128, 2500, dtype, ignore_frac=0.2, seed=35)
    loss_ref, _, rdh, rdw = flce_forward_backward(h, w, y)
    hd = h.to(DEV).requires_grad_(True)
    wd = w.to(DEV).requires_grad_(True)
    loss = LinearCrossEntropyLoss()(hd, wd, y.to(DEV))
    assert loss.dim() == 0
    (2.5 * loss).backward()
    torch.cuda.synchronize()
    tol = TOL[wl.torch_dtype]
    assert abs(float(loss.item()) - loss_ref) <= tol["loss"] * abs(loss_ref)
    _check_grads(to_f64(hd.grad), to_f64(wd.grad), 2.5 * rdh, 2.5 * rdw, wl.torch_dtype, "autograd")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_one_pass(dtype):
    """LinearCrossEntropyLoss(one_pass=True): dH and dW formed in the forward by
    flce_fwd_bwd, scaled by the upstream gradient (2.5) in the backward; the loss
    is bitwise the recompute mode's, the gradients match the oracle's times 2.5,
    only the inputs that require a gradient get one, and a second backward
    through the same graph is refused."""
    wl, (h, w, y) = _case(150, 128, 2500, dtype, ignore_frac=0.2, seed=35)
    loss_ref, _, rdh, rdw = flce_forward_backward(h, w, y)
    hd = h.to(DEV).requires_grad_(True)
    wd = w.to(DEV).requires_grad_(True)
    yd = y.to(DEV)
    loss = LinearCrossEntropyLoss(one_pass=True)(hd, wd, yd)
    loss_rc = LinearCrossEntropyLoss()(hd.detach(), wd.detach(), yd)
    assert loss.dim() == 0 and torch.equal(loss.detach(), loss_rc)
    (2.5 * loss).backward()
    torch.cuda.synchronize()
    tol = TOL[wl.torch_dtype]
    assert abs(float(loss.item()) - loss_ref) <= tol["loss"] * abs(loss_ref)
    _check_grads(to_f64(hd.grad), to_f64(wd.grad), 2.5 * rdh, 2.5 * rdw, wl.torch_dtype, "autograd one pass")

    # upstream gradient 1: the fused call's own dH and dW, untouched
    w2 = w.to(DEV).requires_grad_(True)
    LinearCrossEntropyLoss(one_pass=True)(h.to(DEV), w2, yd).backward()
    _, _, dh1, dw1 = flce.linear_cross_entropy(h.to(DEV), w.to(DEV), yd)
    torch.cuda.synchronize()
    assert torch.equal(w2.grad, dw1)

    # one backward per graph
    h3 = h.to(DEV).requires_grad_(True)
    loss3 = LinearCrossEntropyLoss(one_pass=True)(h3, w.to(DEV), yd)
    loss3.backward(retain_graph=True)
    with pytest.raises(RuntimeError, match="one backward"):
        loss3.backward()


@pytest.mark.parametrize("dtype,count", [("bf16", 4096), ("bf16", 1001), ("f32", 4096), ("f32", 1003)])
def test_scale_in_place(dtype, count):
    """flce_scale: x *= s with the fp32 product rounded to the element type
    (round-to-nearest-even, torch's own conversion), ragged tails included; a
    scale of exactly 1 leaves x bitwise untouched."""
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(count)
    x = torch.randn(count, generator=g).to(td).to(DEV)
    for s in (1.0, 0.5, 3.0, -1e-3):
        y = x.clone()
        flce.scale_(y, torch.tensor([s], dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        want = (x.float() * s).to(td)
        assert torch.equal(y, want if s != 1.0 else x), f"scale {s}"


def test_bwd_single_row_and_tiny_vocab():
    wl, (h, w, y) = _case(1, 16, 5, "bf16", ignore_frac=0.0, seed=36)
    _, lse64 = flce_forward(h, w, y)
    lse32 = torch.from_numpy(lse64.astype(np.float32))
    rdh, rdw = flce_backward_from_lse(h, w, y, lse32.double().numpy())
    dh, dw = flce.linear_cross_entropy_backward(h.to(DEV), w.to(DEV), y.to(DEV), lse32.to(DEV))
    torch.cuda.synchronize()
    _check_grads(to_f64(dh), to_f64(dw), rdh, rdw, torch.bfloat16, "bwd 1x16x5")


@pytest.mark.slow
def test_bwd_llama3_8b_head_full_size():
    """flce_bwd at the Llama-3 head's size from the oracle's full-forward LSE (fp64,
    rounded to fp32), upstream gradient 0.5: dH on sampled token rows and dW on
    sampled vocabulary rows against the oracle, which uses the same LSE."""
    import os
    from oracle import flce_dw_rows, flce_rows
    from workloads import CONFIGS
    wl = CONFIGS["llama3_8b_head"]
    say(f"[bwd] llama3 8b head full size n={wl.n} d={wl.d} v={wl.v}")
    h, w, y = make_inputs(wl)
    w64 = to_f64(w)
    workers = min(16, len(os.sched_getaffinity(0)))
    _, lse64 = flce_forward(h, w64, y, reduction=wl.reduction, workers=workers)
    lse32 = lse64.astype(np.float32)
    g_up = 0.5
    go = torch.tensor([g_up], dtype=torch.float32, device=DEV)
    dh, dw = flce.linear_cross_entropy_backward(h.to(DEV), w.to(DEV), y.to(DEV), torch.from_numpy(lse32).to(DEV), go,
                                                reduction=wl.reduction)
    torch.cuda.synchronize()
    rng = np.random.default_rng(91)
    rows = sorted({0, 4095, 4096, wl.n - 1, *(int(r) for r in rng.choice(wl.n, 12, replace=False))})
    _, rdh = flce_rows(h, w64, y, rows, reduction=wl.reduction)
    cols = sorted({0, wl.v - 1, *(int(c) for c in rng.choice(wl.v, 10, replace=False))})
    rdw = flce_dw_rows(h, w64, y, lse32.astype(np.float64), cols, reduction=wl.reduction)
    e_dh = rel_max(to_f64(dh[torch.tensor(rows, device=DEV)]), g_up * rdh)
    e_dw = rel_max(to_f64(dw[torch.tensor(cols, device=DEV)]), g_up * rdw)
    say(f"  sampled dH rel {e_dh:.2e}, dW rel {e_dw:.2e}")
    tol = TOL[torch.bfloat16]["grad"]
    assert e_dh <= tol and e_dw <= tol


@pytest.mark.slow
@pytest.mark.parametrize("path,chunk,chunks", [("fused", "1280", 7), ("split", "1152", 8)])
def test_paired_chunks_at_scale(monkeypatch, path, chunk, chunks):
    """Chunk pairs over many interior tiles (n = 8192, d = 1024, v = 32000, bf16):
    the fused call with seven chunks (three pairs and a lone last chunk) against the
    full oracle, and the backward from the oracle's LSE with eight chunks (the last
    pair ragged) against the oracle's backward from that LSE."""
    from oracle import flce_forward_backward
    from workloads import Workload
    wl = Workload(f"paired_{path}", 8192, 1024, 32000, "bf16", 0.05, "uniform", 0.05, "mean", seed=95)
    h, w, y = make_inputs(wl, threads=8)
    monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    p = flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16, 1)
    assert (p["num_chunks"], p["dw_pairs"]) == (chunks, 1)
    say(f"[bwd] chunk pairs at scale, {path}: {chunks} chunks of {chunk} rows")
    if path == "fused":
        rl, rlse, rdh, rdw = flce_forward_backward(h, w, y)
        loss, lse, dh, dw = flce.linear_cross_entropy(h.to(DEV), w.to(DEV), y.to(DEV))
        torch.cuda.synchronize()
        assert abs(float(loss.item()) - rl) <= TOL[torch.bfloat16]["loss"] * abs(rl)
    else:
        _, lse64 = flce_forward(h, w, y)
        lse32 = lse64.astype(np.float32)
        rdh, rdw = flce_backward_from_lse(h, w, y, lse32.astype(np.float64), grad_out=0.5)
        go = torch.tensor([0.5], dtype=torch.float32, device=DEV)
        dh, dw = flce.linear_cross_entropy_backward(h.to(DEV), w.to(DEV), y.to(DEV), torch.from_numpy(lse32).to(DEV), go)
        torch.cuda.synchronize()
    _check_grads(to_f64(dh), to_f64(dw), rdh, rdw, torch.bfloat16, f"paired {path}")
