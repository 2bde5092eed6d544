"""Parity of the vocabulary-split path (flce_fwd_shard, flce_merge_shards,
flce_bwd_shard, flce_sum_parts) with the oracle.

Each shard's partial LSE and target logit are compared with the oracle's
partials for the same shard; the merge is fed the oracle's partials (fp32) and
compared with the oracle's merge; the whole split path is compared with the
oracle's unsharded forward and backward.  At the Llama-3 head's full size with
eight shards (the shard shape of an eight-way vocabulary-parallel head) the
loss and every LSE are checked against the oracle's full forward, dH and dW on
sampled rows.
"""
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import (flce_dw_rows, flce_forward, flce_forward_backward, flce_rows, merge_vocab_shards,
                    vocab_shard_partials)
from workloads import CONFIGS, Workload, make_inputs

from gpu_helpers import TOL, rel_max, rel_scalar, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WORKERS = min(16, len(os.sched_getaffinity(0)))


def _case(n, d, v, dtype, ignore_frac=0.1, reduction="mean", seed=0):
    wl = Workload(f"vs_{n}_{d}_{v}", n, d, v, dtype, 0.1, "uniform", ignore_frac, reduction, seed=seed)
    return wl, make_inputs(wl, threads=4)


def _lse_err(a, b):
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shard_partials(dtype):
    n, d, v = 70, 136, 1500
    wl, (h, w, y) = _case(n, d, v, dtype, seed=61)
    y[3] = 600                                   # a label at a shard's first column
    y[4] = 599                                   # and one at the previous shard's last
    tol = TOL[wl.torch_dtype]
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    dt = flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32
    for a, b in [(0, 17), (17, 600), (600, 1500)]:
        say(f"[vocab split] partials {dtype} shard [{a}, {b})")
        lp = torch.empty(n, dtype=torch.float32, device=DEV)
        zp = torch.empty(n, dtype=torch.float32, device=DEV)
        st = flce.flce_fwd_shard(hd, wd[a:b], yd, n, d, b - a, a, dt, -100, lp, zp, torch.cuda.current_stream())
        assert st == flce.FLCE_OK
        torch.cuda.synchronize()
        rlp, rzp = vocab_shard_partials(h, w[a:b], y, a, v_total=v)
        assert _lse_err(to_f64(lp), rlp) <= tol["loss"]
        zg = to_f64(zp)
        assert np.all(zg[rzp == 0.0] == 0.0), "rows whose label is outside the shard must read 0"
        assert rel_max(zg, rzp) <= tol["loss"]


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_merge_from_oracle_partials(reduction):
    n, d, v = 300, 64, 900
    _, (h, w, y) = _case(n, d, v, "f32", reduction=reduction, seed=62)
    cuts = [0, 100, 101, 512, 900]
    parts = [vocab_shard_partials(h, w[a:b], y, a) for a, b in zip(cuts[:-1], cuts[1:])]
    rloss, rlse = merge_vocab_shards([p[0] for p in parts], [p[1] for p in parts], y, reduction=reduction)
    say(f"[vocab split] merge of oracle partials, {len(parts)} shards, {reduction}")
    lp = torch.tensor(np.stack([p[0] for p in parts]).astype(np.float32), device=DEV)
    zp = torch.tensor(np.stack([p[1] for p in parts]).astype(np.float32), device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    lse = torch.empty(n, dtype=torch.float32, device=DEV)
    st = flce.flce_merge_shards(lp, zp, len(parts), y.to(DEV), n, -100,
                                flce.FLCE_MEAN if reduction == "mean" else flce.FLCE_SUM, loss, lse,
                                torch.cuda.current_stream())
    assert st == flce.FLCE_OK
    torch.cuda.synchronize()
    assert rel_scalar(float(loss.item()), rloss) <= 1e-5
    assert _lse_err(to_f64(lse), rlse) <= 1e-6


CASES = [
    ((64, 72, 300), "f32", "mean", [(0, 150), (150, 300)]),
    ((37, 72, 1001), "bf16", "mean", None),                # two shards by default
    ((37, 72, 1001), "f32", "sum", [(0, 17), (17, 700), (700, 1001)]),
    ((513, 520, 2100), "bf16", "mean", [(0, 256), (256, 1024), (1024, 2100)]),
    ((300, 256, 20000), "bf16", "sum", [(0, 9984), (9984, 20000)]),
]


@pytest.mark.parametrize("shape,dtype,reduction,shards", CASES)
def test_vocab_split_end_to_end(shape, dtype, reduction, shards):
    n, d, v = shape
    wl, (h, w, y) = _case(n, d, v, dtype, reduction=reduction, seed=63 + n)
    say(f"[vocab split] end to end n={n} d={d} v={v} {dtype} {reduction} shards={shards}")
    rloss, rlse, rdh, rdw = flce_forward_backward(h, w, y, reduction=reduction)
    g_up = 0.5
    go = torch.tensor([g_up], dtype=torch.float32, device=DEV)
    loss, lse, dh, dw = flce.linear_cross_entropy_vocab_split(h.to(DEV), w.to(DEV), y.to(DEV), reduction=reduction,
                                                              grad_out=go, shards=shards)
    torch.cuda.synchronize()
    tol = TOL[wl.torch_dtype]
    e = dict(loss=rel_scalar(float(loss.item()), rloss), lse=_lse_err(to_f64(lse), rlse),
             dh=rel_max(to_f64(dh), g_up * rdh), dw=rel_max(to_f64(dw), g_up * rdw))
    say(f"  errors {e}")
    assert e["loss"] <= tol["loss"] and e["lse"] <= tol["loss"]
    assert e["dh"] <= tol["grad"] and e["dw"] <= tol["grad"]
    ign = (y == -100).numpy()
    assert np.all(to_f64(dh)[ign] == 0.0)


@pytest.mark.slow
def test_vocab_split_llama3_8b_head_eight_shards():
    wl = CONFIGS["llama3_8b_head"]
    say(f"[vocab split] llama3 8b head, 8 shards: n={wl.n} d={wl.d} v={wl.v}")
    h, w, y = make_inputs(wl)
    loss, lse, dh, dw = flce.linear_cross_entropy_vocab_split(h.to(DEV), w.to(DEV), y.to(DEV), num_shards=8,
                                                              reduction=wl.reduction)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    w64 = to_f64(w)
    rloss, rlse = flce_forward(h, w64, y, reduction=wl.reduction, workers=WORKERS)
    lse_h = to_f64(lse)
    e_loss, e_lse = rel_scalar(float(loss.item()), rloss), _lse_err(lse_h, rlse)
    say(f"  loss rel {e_loss:.2e}, max lse rel {e_lse:.2e}")
    assert e_loss <= tol["loss"] and e_lse <= tol["loss"]
    rng = np.random.default_rng(77)
    rows = sorted({0, wl.n - 1, *(int(r) for r in rng.choice(wl.n, 12, replace=False))})
    _, rdh = flce_rows(h, w64, y, rows, reduction=wl.reduction)
    e_dh = rel_max(to_f64(dh[torch.tensor(rows, device=DEV)]), rdh)
    # vocabulary rows at the shard edges and a few label ids
    edges = [b for _, b in flce.vocab_shard_bounds(wl.v, 8)][:-1]
    cols = sorted({0, wl.v - 1, *(e - 1 for e in edges), *edges, *(int(c) for c in rng.choice(wl.v, 6, replace=False))})
    rdw = flce_dw_rows(h, w64, y, rlse, cols, reduction=wl.reduction)
    e_dw = rel_max(to_f64(dw[torch.tensor(cols, device=DEV)]), rdw)
    say(f"  sampled dH rel {e_dh:.2e}, dW rel {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accumulated_dh_equals_the_summed_parts(dtype):
    """flce_bwd_shard_accumulate adds each shard's dH term into one fp32 sum: the
    result equals the separate terms summed in shard order by flce_sum_parts (to
    fp32 rounding, as split reductions may associate differently), and each
    shard's dW rows are the same either way."""
    n, d, v = 300, 256, 2500
    wl, (h, w, y) = _case(n, d, v, dtype, seed=71)
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    shards = [(0, 700), (700, 1800), (1800, 2500)]
    code = flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32
    _, lse, _, _ = flce.linear_cross_entropy(hd, wd, yd)
    s = torch.cuda.current_stream()
    parts = torch.full((len(shards), n, d), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((n, d), float("nan"), dtype=torch.float32, device=DEV)
    dw_a, dw_b = torch.empty_like(wd), torch.empty_like(wd)
    for q, (a, b) in enumerate(shards):
        assert flce.flce_bwd_shard(hd, wd[a:b], yd, lse, None, n, d, b - a, a, code, -100, flce.FLCE_MEAN, parts[q],
                                   dw_a[a:b], s) == flce.FLCE_OK
        call = flce.flce_bwd_shard if q == 0 else flce.flce_bwd_shard_accumulate
        assert call(hd, wd[a:b], yd, lse, None, n, d, b - a, a, code, -100, flce.FLCE_MEAN, acc, dw_b[a:b],
                    s) == flce.FLCE_OK
    summed = torch.empty(n, d, dtype=torch.float32, device=DEV)
    assert flce.flce_sum_parts(parts, len(shards), n * d, flce.FLCE_F32, summed, s) == flce.FLCE_OK
    torch.cuda.synchronize()
    assert torch.isfinite(acc).all()
    err = float(((acc - summed).abs().max() / summed.abs().max()).item())
    say(f"[vocab split] accumulated dH {dtype}: max diff {err:.2e} of the largest entry")
    assert err <= 1e-6
    assert torch.equal(dw_a, dw_b)
