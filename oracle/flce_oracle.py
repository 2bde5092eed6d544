"""Oracle for fused linear cross-entropy, forward and backward (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import or
call this module.  It shares no code with the HIP library and imports nothing
from it.

It is the plain, materialising definition of what the fused kernels compute,
written from the pages:

* logits ``Z = H . W^T`` over the whole vocabulary -- the un-fused path of the
  blog page "Liger Kernel: Fused Triton Kernels for LLM Training", section
  "The Problem: The Logits Memory Wall" (unembedding projection, logits
  tensor materialised);
* per-row log-sum-exp ``LSE(z) = m + log(sum_j exp(z_j - m))`` with
  ``m = max_j z_j`` -- same page, section "1. Fused Linear Cross-Entropy with
  Online LogSumExp", step 3;
* the target logit ``z_y`` -- same section, step 4; the token NLL is
  ``LSE - z_y``;
* ``dL/dz_j = P(z_j) - 1[j = y]`` with ``P(z_j) = exp(z_j - LSE)``,
  ``dL/dH = (dL/dZ) . W`` and ``dL/dW = (dL/dZ)^T . H`` -- same page, section
  "2. In-Kernel Gradient Computation During the Backward Pass" (the softmax
  there carries a denominator that is identically 1 and is dropped here);
* the backward from the saved per-token LSE alone, recomputing the tile
  logits -- blog page, section "2. In-Kernel Gradient Computation During the
  Backward Pass" (the forward keeps only the LSE; the backward recomputes the
  logits and forms the softmax from it); the gradient of an upstream scalar
  ``g . loss`` is ``g`` times the loss gradient;
* cross-entropy on logits that are already materialised (the
  ``LigerCrossEntropyLoss`` example of the lecture page, a drop-in for
  PyTorch's loss on a ``[B*S, vocab]`` logits view): the same LSE, target and
  gradient formulas applied to a given ``[N, V]`` logits array;
* the vocabulary split the lecture page leaves open for vocabularies of a
  million ids ("GPU MODE lecture 028 - Liger Kernel", open questions): each
  contiguous shard of W's rows yields a per-row partial LSE and, where the
  label falls in it, the target logit; the whole-vocabulary LSE is the LSE of
  the partial LSEs (the merge of the blog page's section "1. Fused Linear
  Cross-Entropy with Online LogSumExp", step 3, taken over shards instead of
  tiles), and a shard's gradient is the softmax-minus-one-hot formula on its
  own columns with the merged LSE;
* FP8 inputs, which the lecture page raises only as an open question (FP8
  training on newer GPUs) without a method: the forward of e4m3-quantised H
  and W with one scale per row is the forward of the dequantised matrices,
  ``z_ij = s_h[i] s_w[j] sum_k q_h[i, k] q_w[j, k]``; e4m3 is the OCP 8-bit
  float with 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa bits,
  subnormals at exponent 0 and no infinities (S.1111.111 is NaN); the FP8
  backward is the gradient of that same loss with respect to the dequantised
  H and W, from the saved LSE (the blog page's backward section applied to
  the dequantised matrices);
* ``reduction="mean"`` as in the loss module call on the lecture page
  ("GPU MODE lecture 028 - Liger Kernel", the LigerCrossEntropyLoss example);
  the mean is taken over the rows whose label is not ``ignore_index``, and a
  mean over zero valid rows is defined as 0 (loss and gradients), a reading of
  the pages, which are silent on it.

Everything is computed in float64 from the exact float64 images of the inputs
(bf16 and fp32 values convert exactly).  The row blocking below only bounds
host memory; every block sees the full vocabulary, so no online merging
happens here.

Every public function is pinned, in ``tests/test_oracle_pins.py``, to
something other than itself: closed forms, brute-force loops, finite
differences, torch's float64 cross-entropy and autograd, the figures the blog
page prints, and planted-mistake checks.  None is left unpinned.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def _as_f64(x) -> np.ndarray:
    """Exact float64 image of a float32/bf16/float64 array or CPU torch tensor."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype, go through float32 (exact)
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _as_labels(y) -> np.ndarray:
    if hasattr(y, "detach"):
        y = y.detach().to("cpu").numpy()
    return np.asarray(y, dtype=np.int64)


def valid_rows(labels, v: int, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Boolean mask of rows that count toward the loss.

    A label must be ``ignore_index`` or lie in ``[0, v)``; anything else is a
    caller error and raises ``ValueError``.
    """
    y = _as_labels(labels)
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= v))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"label {int(y[i])} at row {i} is outside [0, {v}) and is not ignore_index")
    return valid


def reduction_scale(n_valid: int, reduction: str) -> float:
    """Factor applied to every valid row's NLL and gradient: 1/n_valid for mean, 1 for sum."""
    if reduction == "mean":
        return 1.0 / n_valid if n_valid > 0 else 0.0
    if reduction == "sum":
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def log_sum_exp(z: np.ndarray) -> np.ndarray:
    """Row-wise LSE(z) = m + log(sum_j exp(z_j - m)), m = max_j z_j."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def flce_forward(h, w, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                 block_rows: int = 1024, workers: int = 1):
    """Loss (float) and per-row LSE [N] (float64) of softmax(H W^T) against the labels.

    ``workers`` > 1 evaluates independent row blocks on that many threads; the
    arithmetic of every block is unchanged.
    """
    hd, wd, y = _as_f64(h), _as_f64(w), _as_labels(labels)
    n, v = hd.shape[0], wd.shape[0]
    valid = valid_rows(y, v, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    lse = np.empty(n, dtype=np.float64)
    nll = np.zeros(n, dtype=np.float64)

    def block(r0):
        r1 = min(n, r0 + block_rows)
        z = hd[r0:r1] @ wd.T
        lse[r0:r1] = log_sum_exp(z)
        rows = np.flatnonzero(valid[r0:r1])
        nll[r0 + rows] = lse[r0 + rows] - z[rows, y[r0 + rows]]

    starts = range(0, n, block_rows)
    if workers > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(block, starts))
    else:
        for r0 in starts:
            block(r0)
    return float(scale * nll.sum()), lse


def flce_forward_backward(h, w, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                          block_rows: int = 1024):
    """Return (loss, lse[N], dH[N, D], dW[V, D]), all float64.

    The gradients are those of the returned loss with an upstream gradient of 1.
    Ignored rows contribute nothing to the loss, have a zero dH row and add
    nothing to dW; their LSE is still reported.
    """
    hd, wd, y = _as_f64(h), _as_f64(w), _as_labels(labels)
    n, d = hd.shape
    v = wd.shape[0]
    if wd.shape[1] != d:
        raise ValueError("H and W disagree on the hidden size")
    valid = valid_rows(y, v, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    lse = np.empty(n, dtype=np.float64)
    nll = np.zeros(n, dtype=np.float64)
    dh = np.zeros((n, d), dtype=np.float64)
    dw = np.zeros((v, d), dtype=np.float64)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        z = hd[r0:r1] @ wd.T                       # logits block, all V columns
        lse_b = log_sum_exp(z)
        lse[r0:r1] = lse_b
        rows = np.flatnonzero(valid[r0:r1])
        tgt = y[r0 + rows]
        nll[r0 + rows] = lse_b[rows] - z[rows, tgt]
        g = np.exp(z - lse_b[:, None])             # softmax P(z)
        g[rows, tgt] -= 1.0                        # P - onehot
        g[~valid[r0:r1]] = 0.0                     # ignored rows carry no gradient
        g *= scale
        dh[r0:r1] = g @ wd                         # dL/dH = (dL/dZ) W
        dw += g.T @ hd[r0:r1]                      # dL/dW = (dL/dZ)^T H
    return float(scale * nll.sum()), lse, dh, dw


def flce_rows(h, w, labels, rows, ignore_index: int = IGNORE_INDEX, reduction: str = "mean"):
    """LSE and dH for selected rows only, at any problem size.

    Each row's LSE and gradient depend only on that row's logits and on the
    global valid count (for the mean), so they can be computed one by one.
    Returns (lse[len(rows)], dH[len(rows), D]).
    """
    wd, y = _as_f64(w), _as_labels(labels)
    v = wd.shape[0]
    valid = valid_rows(y, v, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    rows = np.asarray(rows, dtype=np.int64)
    if hasattr(h, "detach"):
        import torch
        hr = _as_f64(h[torch.as_tensor(rows)])
    else:
        hr = _as_f64(np.asarray(h)[rows])
    z = hr @ wd.T
    lse = log_sum_exp(z)
    g = np.exp(z - lse[:, None])
    vr = valid[rows]
    idx = np.flatnonzero(vr)
    g[idx, y[rows[idx]]] -= 1.0
    g[~vr] = 0.0
    g *= scale
    return lse, g @ wd


def flce_dw_rows(h, w, labels, lse, vocab_rows, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                 block_rows: int = 8192):
    """dW rows for selected vocabulary ids, at any problem size.

    dW_j = sum_i scale_i * (exp(z_ij - lse_i) - [y_i = j]) * H_i needs every
    row's LSE, which the caller obtains from ``flce_forward`` (never from the
    code under test).  Returns [len(vocab_rows), D] float64.
    """
    y = _as_labels(labels)
    cols = np.asarray(vocab_rows, dtype=np.int64)
    if hasattr(w, "detach"):
        import torch
        wj = _as_f64(w[torch.as_tensor(cols)])
        v = w.shape[0]
    else:
        wj = _as_f64(np.asarray(w)[cols])
        v = np.asarray(w).shape[0]
    valid = valid_rows(y, v, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    lse = np.asarray(lse, dtype=np.float64)
    n = y.shape[0]
    out = np.zeros((cols.size, wj.shape[1]), dtype=np.float64)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        hb = _as_f64(h[r0:r1])
        g = np.exp(hb @ wj.T - lse[r0:r1, None])          # softmax columns j, [rows, |J|]
        g -= (y[r0:r1, None] == cols[None, :])             # one-hot
        g[~valid[r0:r1]] = 0.0
        g *= scale
        out += g.T @ hb
    return out


def flce_backward_from_lse(h, w, labels, lse, grad_out: float = 1.0, ignore_index: int = IGNORE_INDEX,
                           reduction: str = "mean", block_rows: int = 1024):
    """(dH[N, D], dW[V, D]) float64 of ``grad_out * loss`` from the saved per-row LSE.

    The logits are recomputed block by block and the softmax is formed as
    exp(z - lse) from the LSE handed in, as the backward pass of the blog page
    does; with the forward's LSE this equals ``flce_forward_backward``'s
    gradients times ``grad_out``.
    """
    hd, wd, y = _as_f64(h), _as_f64(w), _as_labels(labels)
    n, d = hd.shape
    v = wd.shape[0]
    lse = np.asarray(lse, dtype=np.float64)
    valid = valid_rows(y, v, ignore_index)
    scale = float(grad_out) * reduction_scale(int(valid.sum()), reduction)
    dh = np.zeros((n, d), dtype=np.float64)
    dw = np.zeros((v, d), dtype=np.float64)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        z = hd[r0:r1] @ wd.T                       # recomputed logits block
        g = np.exp(z - lse[r0:r1, None])           # softmax from the saved LSE
        rows = np.flatnonzero(valid[r0:r1])
        g[rows, y[r0 + rows]] -= 1.0
        g[~valid[r0:r1]] = 0.0
        g *= scale
        dh[r0:r1] = g @ wd
        dw += g.T @ hd[r0:r1]
    return dh, dw


def ce_on_logits(z, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean"):
    """Cross-entropy on given logits: (loss, lse[N], dL/dz[N, V]), float64."""
    zd, y = _as_f64(z), _as_labels(labels)
    n, v = zd.shape
    valid = valid_rows(y, v, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    lse = log_sum_exp(zd)
    rows = np.flatnonzero(valid)
    loss = scale * float(np.sum(lse[rows] - zd[rows, y[rows]]))
    g = np.exp(zd - lse[:, None])
    g[rows, y[rows]] -= 1.0
    g[~valid] = 0.0
    g *= scale
    return loss, lse, g


def vocab_shard_partials(h, w_shard, labels, v_first: int, ignore_index: int = IGNORE_INDEX,
                         v_total: int | None = None):
    """One vocabulary shard's partials: (lse_part[N], zy_part[N]) float64.

    ``w_shard`` holds the rows ``v_first .. v_first + v_shard - 1`` of W.
    lse_part is the log-sum-exp of the row's logits over the shard's columns;
    zy_part is the target logit when the row's label lies in the shard, else
    0 (also 0 for ignored rows).  Labels are whole-vocabulary ids, checked
    against ``v_total`` when given.
    """
    hd, wd, y = _as_f64(h), _as_f64(w_shard), _as_labels(labels)
    v_shard = wd.shape[0]
    valid = valid_rows(y, v_total, ignore_index) if v_total is not None else y != ignore_index
    z = hd @ wd.T                                   # the shard's logits, all rows
    lse_part = log_sum_exp(z)
    local = y - int(v_first)
    here = np.flatnonzero(valid & (local >= 0) & (local < v_shard))
    zy_part = np.zeros(y.shape[0], dtype=np.float64)
    zy_part[here] = z[here, local[here]]
    return lse_part, zy_part


def merge_vocab_shards(lse_parts, zy_parts, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean"):
    """(loss, lse[N]) float64 from the shards' partials ([shards, N] each).

    lse = log sum_q exp(lse_q) (largest partial factored out first); the
    target logit is the one shard's nonzero entry, i.e. the sum over shards;
    the loss reduces lse - z_y over the valid rows.
    """
    lp = np.asarray(lse_parts, dtype=np.float64)
    zp = np.asarray(zy_parts, dtype=np.float64)
    y = _as_labels(labels)
    valid = y != ignore_index
    scale = reduction_scale(int(valid.sum()), reduction)
    m = lp.max(axis=0)
    lse = m + np.log(np.exp(lp - m[None, :]).sum(axis=0))
    zy = zp.sum(axis=0)
    loss = scale * float(np.sum(lse[valid] - zy[valid]))
    return loss, lse


def vocab_shard_backward(h, w_shard, labels, lse, v_first: int, grad_out: float = 1.0,
                         ignore_index: int = IGNORE_INDEX, reduction: str = "mean"):
    """(dH_part[N, D], dW_shard[v_shard, D]) float64 of ``grad_out * loss`` for one shard.

    G_q = (exp(z_q - lse) - onehot) * scale * grad_out over the shard's columns
    only, with the whole-vocabulary LSE; dH = sum over shards of G_q W_q and
    dW's rows of the shard are G_q^T H.
    """
    hd, wd, y = _as_f64(h), _as_f64(w_shard), _as_labels(labels)
    v_shard = wd.shape[0]
    lse = np.asarray(lse, dtype=np.float64)
    valid = y != ignore_index
    scale = float(grad_out) * reduction_scale(int(valid.sum()), reduction)
    g = np.exp(hd @ wd.T - lse[:, None])
    local = y - int(v_first)
    here = np.flatnonzero(valid & (local >= 0) & (local < v_shard))
    g[here, local[here]] -= 1.0
    g[~valid] = 0.0
    g *= scale
    return g @ wd, g.T @ hd


def decode_e4m3(codes) -> np.ndarray:
    """float64 values of OCP e4m3 bytes (any shape), from the format definition.

    Exponent field e, mantissa field m: e = 0 is subnormal, m/8 * 2^-6; else
    (1 + m/8) * 2^(e - 7); the code with e = 15 and m = 7 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    out[(e == 15) & ((c & 0x7) == 7)] = np.nan
    return out


def flce_forward_fp8(h_q, h_scale, w_q, w_scale, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                     block_rows: int = 1024, workers: int = 1):
    """Loss and LSE[N] (float64) of the forward on e4m3 H and W with one fp32 scale per row."""
    def codes(x):
        if hasattr(x, "detach"):
            import torch
            x = x.detach().to("cpu").contiguous().view(torch.uint8).numpy()
        return np.asarray(x, dtype=np.uint8)
    h = decode_e4m3(codes(h_q)) * _as_f64(h_scale)[:, None]
    w = decode_e4m3(codes(w_q)) * _as_f64(w_scale)[:, None]
    return flce_forward(h, w, labels, ignore_index=ignore_index, reduction=reduction, block_rows=block_rows,
                        workers=workers)


def flce_backward_fp8(h_q, h_scale, w_q, w_scale, labels, lse, grad_out: float = 1.0,
                      ignore_index: int = IGNORE_INDEX, reduction: str = "mean"):
    """(dH, dW) float64 of ``grad_out * loss`` with respect to the dequantised H and W
    of e4m3 inputs with per-row scales, from the saved per-row LSE."""
    def codes(x):
        if hasattr(x, "detach"):
            import torch
            x = x.detach().to("cpu").contiguous().view(torch.uint8).numpy()
        return np.asarray(x, dtype=np.uint8)
    h = decode_e4m3(codes(h_q)) * _as_f64(h_scale)[:, None]
    w = decode_e4m3(codes(w_q)) * _as_f64(w_scale)[:, None]
    return flce_backward_from_lse(h, w, labels, lse, grad_out=grad_out, ignore_index=ignore_index,
                                  reduction=reduction)

