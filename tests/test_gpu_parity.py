"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by
element, at sizes the oracle finishes in seconds; plus the degenerate cases."""
import math
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_forward_backward
from workloads import CONFIGS, Workload, make_inputs

from gpu_helpers import TOL, check, run_lib, say, to_f64

pytestmark = pytest.mark.gpu


def _case(n, d, v, dtype, sigma_w=0.02, ignore_frac=0.1, reduction="mean", seed=0, labels="uniform"):
    wl = Workload(f"case_{n}_{d}_{v}", n, d, v, dtype, sigma_w, labels, ignore_frac, reduction, seed=seed)
    return wl, make_inputs(wl, threads=4)


def _parity(wl, inputs, what):
    h, w, y = inputs
    say(f"[parity] {what}: n={wl.n} d={wl.d} v={wl.v} {wl.dtype} {wl.reduction}")
    gpu = run_lib(h, w, y, wl.reduction)
    ref = flce_forward_backward(h, w, y, reduction=wl.reduction)
    return check(gpu, ref, wl.torch_dtype, what)


def test_tiny_f32_config():
    wl = CONFIGS["tiny_f32"]
    _parity(wl, make_inputs(wl), "tiny_f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_odd_shapes(dtype, reduction):
    wl, inp = _case(37, 72, 1001, dtype, sigma_w=0.3, reduction=reduction, seed=11)
    _parity(wl, inp, f"odd {dtype} {reduction}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_tile_ragged(dtype):
    wl, inp = _case(700, 264, 3000, dtype, sigma_w=0.1, reduction="sum", seed=12)
    _parity(wl, inp, f"ragged {dtype}")


def test_blog_simulation_regime_f32():
    """N=128, D=512, V=4096 with W ~ N(0, 1): logits with sigma ~ 22 (the blog's
    fused-vs-unfused numerical check uses these sizes and unit-variance weights)."""
    wl, inp = _case(128, 512, 4096, "f32", sigma_w=1.0, ignore_frac=0.0, seed=13)
    _parity(wl, inp, "blog regime")


def test_large_logits_bf16():
    """W ~ N(0, 0.5^2) at D=4096: |z| beyond 88, where exp overflows in fp32 without max subtraction."""
    wl, inp = _case(96, 4096, 2000, "bf16", sigma_w=0.5, ignore_frac=0.0, seed=14)
    _parity(wl, inp, "large logits")


@pytest.mark.parametrize("chunk", [None, "64"])
def test_folded_factor_flagged_rows(monkeypatch, chunk):
    """The matrix engine's one-pass backward stores each row's P against the
    row's target logit and applies the softmax factor per row (to dH's rows and
    to dW's copy of H).  A row whose target logit lies more than 30 below some
    128-column group's max is flagged and brought to the row max after the
    merge.  W ~ N(0, 0.5^2) at D = 512 gives both kinds of row; chunks of 64
    rows add paired dW launches and a ragged last chunk."""
    n, d, v = 300, 512, 4100
    wl, (h, w, y) = _case(n, d, v, "bf16", sigma_w=0.5, ignore_frac=0.1, seed=31)
    if chunk is not None:
        monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    p = flce.flce_plan_info(n, d, v, flce.FLCE_BF16, 1)
    assert p["folded_factor"] == 1
    # the case holds flagged and unflagged rows (fp64 logits of the bf16 inputs)
    z = h.double().numpy() @ w.double().numpy().T
    zp = np.full((n, (v + 127) // 128 * 128), -np.inf)
    zp[:, :v] = z
    gmax = zp.reshape(n, -1, 128).max(axis=2)
    valid = (y != -100).numpy()
    zy = z[np.arange(n), np.where(valid, y.numpy(), 0)]
    flagged = np.any(gmax - 30.0 > zy[:, None], axis=1) & valid
    assert 0 < int(flagged.sum()) < int(valid.sum())
    _parity(wl, (h, w, y), f"flagged rows, chunk {chunk}")


def test_all_rows_ignored():
    for red in ("mean", "sum"):
        wl, (h, w, y) = _case(64, 128, 500, "f32", sigma_w=0.2, seed=15, reduction=red)
        y[:] = -100
        loss, lse, dh, dw = run_lib(h, w, y, red)
        ref = flce_forward_backward(h, w, y, reduction=red)
        assert loss == 0.0
        assert np.all(dh == 0.0) and np.all(dw == 0.0)
        assert np.max(np.abs(lse - ref[1]) / np.abs(ref[1])) <= 1e-5


def test_all_rows_ignored_bf16():
    """bf16 with the per-row gradient factor: every row ignored gives loss 0, zero
    gradients and the true LSE of every row."""
    for red in ("mean", "sum"):
        wl, (h, w, y) = _case(300, 128, 1500, "bf16", sigma_w=0.2, seed=19, reduction=red)
        y[:] = -100
        assert flce.flce_plan_info(300, 128, 1500, flce.FLCE_BF16, 1)["folded_factor"] == 1
        loss, lse, dh, dw = run_lib(h, w, y, red)
        ref = flce_forward_backward(h, w, y, reduction=red)
        assert loss == 0.0
        assert np.all(dh == 0.0) and np.all(dw == 0.0)
        assert np.max(np.abs(lse - ref[1]) / np.abs(ref[1])) <= TOL[torch.bfloat16]["loss"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_labels_outside_the_vocabulary(dtype):
    """Labels outside [0, v) that are not ignore_index are a caller error the header
    defines: the row counts as valid, with target logit 0 and no one-hot term.  With
    the sum reduction that is the oracle's result with those rows ignored, plus
    lse_i in the loss and softmax_i in G for each of them (computed here in fp64).
    On the bf16 engine such rows have no target reference and take the flagged path."""
    n, d, v = 200, 128, 1000
    wl, (h, w, y) = _case(n, d, v, dtype, sigma_w=0.2, ignore_frac=0.1, seed=37, reduction="sum")
    rng = np.random.default_rng(37)
    oor = rng.choice(np.flatnonzero((y != -100).numpy()), size=24, replace=False)
    y_bad = y.clone()
    y_bad[torch.from_numpy(oor[:12])] = v + 7
    y_bad[torch.from_numpy(oor[12:])] = -5
    y_ign = y.clone()
    y_ign[torch.from_numpy(oor)] = -100
    rloss, rlse, rdh, rdw = flce_forward_backward(h, w, y_ign, reduction="sum")
    hd, wd = to_f64(h), to_f64(w)
    p = np.exp(hd[oor] @ wd.T - rlse[oor, None])            # softmax rows of the out-of-range rows
    rloss = rloss + float(rlse[oor].sum())
    rdh = rdh.copy()
    rdh[oor] = p @ wd
    rdw = rdw + p.T @ hd[oor]
    say(f"[parity] labels outside [0, v): {len(oor)} rows, {dtype}")
    gpu = run_lib(h, w, y_bad, "sum")
    check(gpu, (rloss, rlse, rdh, rdw), wl.torch_dtype, "labels outside the vocabulary")


def test_debug_label_check(monkeypatch):
    """FLCE_CHECK_LABELS=1 makes the binding refuse a label outside [0, v) that is
    not ignore_index (ValueError naming the row) before any library call; unset,
    the call runs with the documented meaning of such a row."""
    wl, (h, w, y) = _case(40, 64, 300, "bf16", sigma_w=0.1, seed=38)
    hd, wd, yd = h.to("cuda:0"), w.to("cuda:0"), y.clone()
    yd[7] = 300
    yd = yd.to("cuda:0")
    flce.linear_cross_entropy(hd, wd, yd)
    monkeypatch.setenv("FLCE_CHECK_LABELS", "1")
    with pytest.raises(ValueError, match="row 7"):
        flce.linear_cross_entropy(hd, wd, yd)
    with pytest.raises(ValueError, match="row 7"):
        flce.linear_cross_entropy_forward(hd, wd, yd)
    with pytest.raises(ValueError, match="row 7"):
        flce.cross_entropy(torch.zeros(40, 300, dtype=torch.bfloat16, device="cuda:0"), yd)
    ok = y.to("cuda:0")
    flce.linear_cross_entropy(hd, wd, ok)                 # valid and ignored labels pass
    torch.cuda.synchronize()


def test_w_zero_closed_form():
    wl, (h, w, y) = _case(80, 64, 300, "f32", seed=16)
    w.zero_()
    loss, lse, dh, dw = run_lib(h, w, y, "mean")
    assert abs(loss - math.log(300)) <= 1e-5 * math.log(300)
    assert np.allclose(lse, math.log(300), rtol=1e-6)
    assert np.all(dh == 0.0)
    check((loss, lse, dh, dw), flce_forward_backward(h, w, y), torch.float32, "W=0")


def test_logit_shift_100_f32():
    """Append a ones column to H and a column of 100 to W: every logit moves by 100.

    Loss, dH[:, :D] and dW[:, :D] must match the unshifted oracle and the LSE
    moves by exactly 100.  The extra dH column equals 100 * sum_j G_ij, whose
    exact value is 0; in fp32 its rounding error is amplified by 100, so it is
    held to that bound (100 * 1e-5 * sum_j |G_ij|, with sum_j |G_ij| <= 2 / n_valid)
    instead of the max-normalised gradient tolerance.
    """
    n, d, v, c = 64, 60, 700, 100.0
    wl, (h, w, y) = _case(n, d, v, "f32", sigma_w=0.3, seed=17)
    h1 = torch.cat([h, torch.ones(n, 1), torch.zeros(n, 3)], dim=1)      # d + 4 keeps 16-byte rows
    w1 = torch.cat([w, torch.full((v, 1), c), torch.zeros(v, 3)], dim=1)
    loss, lse, dh, dw = run_lib(h1, w1, y)
    base = flce_forward_backward(h, w, y)
    shifted = flce_forward_backward(h1, w1, y)
    check((loss, lse - c, dh[:, :d], dw[:, :d]), base, torch.float32, "shift 100 vs unshifted")
    n_valid = int((y != -100).sum())
    assert np.max(np.abs(dh[:, d])) <= c * 1e-5 * 2.0 / n_valid
    g_colsum = shifted[3][:, d]
    assert np.max(np.abs(dw[:, d] - g_colsum)) <= 1e-4 * np.max(np.abs(shifted[3]))
    assert np.all(dh[:, d + 1:] == 0.0) and np.all(dw[:, d + 1:] == 0.0)


@pytest.mark.parametrize("c", [100.0, -100.0])
def test_logit_shift_bf16_folded(c):
    """The shift of every logit by +-100 (a ones column in H, a column of c in W,
    both exact in bf16) on the bf16 path with the per-row factor: the target-logit
    references, the group maxes and the LSE all move by c, and loss, dH[:, :D] and
    dW[:, :D] match the unshifted oracle; the LSE moves by c."""
    n, d, v = 300, 64, 2000
    wl, (h, w, y) = _case(n, d, v, "bf16", sigma_w=0.3, seed=27)
    h1 = torch.cat([h, torch.ones(n, 1, dtype=h.dtype), torch.zeros(n, 7, dtype=h.dtype)], dim=1)
    w1 = torch.cat([w, torch.full((v, 1), c, dtype=w.dtype), torch.zeros(v, 7, dtype=w.dtype)], dim=1)
    assert flce.flce_plan_info(n, d + 8, v, flce.FLCE_BF16, 1)["folded_factor"] == 1
    say(f"[parity] logit shift {c:+.0f}, bf16 folded")
    loss, lse, dh, dw = run_lib(h1, w1, y)
    base = flce_forward_backward(h, w, y)
    check((loss, lse - c, dh[:, :d], dw[:, :d]), base, torch.bfloat16, f"shift {c:+.0f} vs unshifted")


def test_labels_at_vocab_edges():
    wl, (h, w, y) = _case(50, 64, 777, "bf16", sigma_w=0.2, ignore_frac=0.0, seed=18)
    y[0::3] = 0
    y[1::3] = 776
    _parity(wl, (h, w, y), "edge labels")


def test_determinism_and_fwd_agreement():
    wl, (h, w, y) = _case(300, 128, 2500, "bf16", sigma_w=0.1, seed=19)
    a = run_lib(h, w, y)
    b = run_lib(h, w, y)
    assert a[0] == b[0]
    for x, z in zip(a[1:], b[1:]):
        assert np.array_equal(x, z)
    hd, wd, yd = h.cuda(), w.cuda(), y.cuda()
    loss_f, lse_f = flce.linear_cross_entropy_forward(hd, wd, yd)
    torch.cuda.synchronize()
    assert float(loss_f.item()) == a[0]
    assert np.array_equal(to_f64(lse_f), a[1])


@pytest.mark.parametrize("chunk", ["16", "48", "256"])
def test_chunk_size_invariance(monkeypatch, chunk):
    wl, (h, w, y) = _case(260, 96, 1500, "f32", sigma_w=0.2, seed=20)
    ref = flce_forward_backward(h, w, y)
    monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    check(run_lib(h, w, y), ref, torch.float32, f"chunk {chunk}")


# chunk rows -> (chunks, paired): 128 rows give an unpaired first, middle and last
# chunk; 80 rows two pairs, the second ragged; 64 rows a first pair, a middle pair
# and a lone ragged last chunk; 512 rows a single chunk.
CHUNK_MODES = {"128": (3, 0), "80": (4, 1), "64": (5, 1), "512": (1, 0)}


@pytest.mark.parametrize("grad", ["folded", "inplace"])
@pytest.mark.parametrize("chunk", list(CHUNK_MODES))
def test_chunk_modes_bf16(monkeypatch, chunk, grad):
    """The matrix engine's dW accumulation modes on interior 256x256 tiles, chunk by
    chunk and over chunk pairs (one launch reducing over two chunks' rows), with
    the softmax factor applied per row (dW reads the scaled copy of H) or written
    into the stored probabilities in place."""
    wl, inp = _case(300, 256, 1500, "bf16", sigma_w=0.1, seed=25)
    monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    if grad == "inplace":
        monkeypatch.setenv("FLCE_INPLACE_GRAD", "1")
    p = flce.flce_plan_info(300, 256, 1500, flce.FLCE_BF16, 1)
    assert (p["num_chunks"], p["dw_pairs"]) == CHUNK_MODES[chunk]
    assert p["folded_factor"] == int(grad == "folded")
    _parity(wl, inp, f"bf16 chunk {chunk}, {grad}")


def test_ignored_rows_exact_zero_and_isolation():
    wl, (h, w, y) = _case(200, 128, 1200, "bf16", sigma_w=0.1, ignore_frac=0.25, seed=21)
    loss, lse, dh, dw = run_lib(h, w, y)
    ign = (y == -100).numpy()
    assert np.all(dh[ign] == 0.0)
    h2 = h.clone()
    h2[torch.from_numpy(ign)] = 3.0
    loss2, lse2, dh2, dw2 = run_lib(h2, w, y)
    assert loss2 == loss
    assert np.array_equal(dw2, dw)
    assert np.array_equal(dh2, dh)


def test_dw_rows_sum_to_zero():
    wl, (h, w, y) = _case(300, 128, 1000, "f32", sigma_w=0.2, seed=22)
    _, _, _, dw = run_lib(h, w, y)
    assert np.max(np.abs(dw.sum(axis=0))) <= 1e-4 * np.max(np.abs(dw))


def test_dh_split_vocab_bf16():
    """Vocabulary large enough that dH = G.W splits its vocabulary reduction."""
    wl, inp = _case(300, 256, 20000, "bf16", sigma_w=0.05, seed=23)
    assert flce.flce_plan_info(300, 256, 20000, flce.FLCE_BF16, 1)["dh_splits"] > 1
    _parity(wl, inp, "dh split")


@pytest.mark.parametrize("shape", [(513, 520, 2100), (64, 8, 300), (1, 16, 5)])
def test_mfma_tails_bf16(shape):
    """Ragged token, hidden and vocabulary tails of the 256x256x64 tiles."""
    n, d, v = shape
    wl, inp = _case(n, d, v, "bf16", sigma_w=0.1, seed=24)
    _parity(wl, inp, f"tails {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_vocabulary_of_one(dtype):
    """Degenerate vocabulary V = 1: the softmax is identically 1, so every valid
    row's loss is 0, its LSE is its single logit, and both gradients vanish, up
    to the fp32 rounding of exp(z - max) (the matrix engine forms the exponent as
    z log2(e) minus its rounded max, a residual of order 1e-8)."""
    n, d, v = 5, 16, 1
    wl = Workload("v1", n, d, v, dtype, 0.3, "uniform", 0.0, "mean", seed=25)
    h, w, y = make_inputs(wl, threads=1)
    y[3] = -100
    say(f"[parity] vocabulary of one {dtype}")
    loss, lse, dh, dw = run_lib(h, w, y)
    z = to_f64(h) @ to_f64(w).T
    assert abs(loss) <= 1e-6
    assert np.max(np.abs(lse - z[:, 0])) <= TOL[wl.torch_dtype]["loss"] * max(1.0, float(np.max(np.abs(z))))
    assert np.max(np.abs(dh)) <= 1e-6 * max(1.0, float(np.max(np.abs(to_f64(w)))))
    assert np.max(np.abs(dw)) <= 1e-6 * max(1.0, float(np.max(np.abs(to_f64(h)))))
