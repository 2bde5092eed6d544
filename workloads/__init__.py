"""Seeded synthetic inputs for fused linear cross-entropy.

This module holds no part of the loss arithmetic.  It only draws the inputs
that the oracle and the HIP path both consume, so that the two sides see
bit-identical values:

* hidden states ``H[N, D]``  ~ N(0, 1)
* LM-head weight ``W[V, D]`` ~ N(0, sigma_w^2)
* integer labels ``y[N]`` (uniform or truncated Zipf over vocabulary ids)
  with an exact count of rows set to ``ignore_index`` (-100).

Shapes follow the LM heads the pages talk about: the Llama-3 8B head
(D = 4096, V = 128256; "Liger Kernel: Fused Triton Kernels for LLM Training",
section "The 128k Vocabulary Explosion") and a Qwen2-style ~152K vocabulary
("GPU MODE lecture 028 - Liger Kernel", practice step 8).  No dataset items
are reproduced: every value is drawn from the seeded generators below.

Normals are drawn in float32 with numpy's PCG64 and then rounded to the
config dtype with round-to-nearest-even (``torch.Tensor.to``).  Large arrays
are drawn in fixed row blocks, each with its own child seed, so the values do
not depend on how many threads draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

IGNORE_INDEX = -100
_BLOCK_ROWS = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic input recipe."""

    name: str
    n: int
    d: int
    v: int
    dtype: str               # "f32" or "bf16"
    sigma_w: float
    labels: str               # "uniform" or "zipf1.1"
    ignore_frac: float        # exact count round(frac * n), seeded permutation
    reduction: str            # "mean" or "sum"
    ignored_rows: Optional[tuple] = None   # explicit [lo, hi) all-ignored block
    seed: int = 0             # k: H uses 1000+k, W 2000+k, labels 3000+k

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the build is measured and checked on.
CONFIGS = {
    "tiny_f32": Workload("tiny_f32", 256, 512, 4096, "f32", 0.02, "uniform", 0.10, "mean", seed=1),
    "llama3_8b_head": Workload("llama3_8b_head", 8192, 4096, 128256, "bf16", 0.02, "uniform", 0.05, "mean", seed=2),
    "qwen2_head": Workload("qwen2_head", 4096, 3584, 151936, "bf16", 0.02, "zipf1.1", 0.05, "mean", seed=3),
    "long_context": Workload("long_context", 32768, 4096, 128256, "bf16", 0.02, "uniform", 0.02, "sum", seed=4),
    "stability_stress": Workload("stability_stress", 16384, 4096, 32000, "bf16", 0.5, "uniform", 0.0, "mean",
                                 ignored_rows=(4096, 8192), seed=5),
}


def _normal_rows(seed: int, rows: int, cols: int, sigma: float, threads: Optional[int] = None) -> np.ndarray:
    """float32 N(0, sigma^2) array of shape [rows, cols], drawn in row blocks."""
    out = np.empty((rows, cols), dtype=np.float32)
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS
    children = np.random.SeedSequence(seed).spawn(max(nblk, 1))

    def fill(b):
        lo = b * _BLOCK_ROWS
        hi = min(rows, lo + _BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(children[b]))
        blk = out[lo:hi]
        g.standard_normal(out=blk, dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if nblk <= 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def zipf_probabilities(v: int, s: float = 1.1) -> np.ndarray:
    """P(id = k) proportional to (k + 1)^-s for k in [0, v): Zipf truncated to the vocabulary."""
    w = np.arange(1, v + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def make_labels(wl: Workload) -> np.ndarray:
    rng = np.random.default_rng(3000 + wl.seed)
    if wl.labels == "uniform":
        y = rng.integers(0, wl.v, size=wl.n, dtype=np.int64)
    elif wl.labels.startswith("zipf"):
        s = float(wl.labels[4:])
        cdf = np.cumsum(zipf_probabilities(wl.v, s))
        u = rng.random(wl.n)
        y = np.minimum(np.searchsorted(cdf, u * cdf[-1], side="right"), wl.v - 1).astype(np.int64)
    else:
        raise ValueError(f"unknown label law {wl.labels!r}")
    k = int(round(wl.ignore_frac * wl.n))
    if k:
        y[rng.permutation(wl.n)[:k]] = IGNORE_INDEX
    if wl.ignored_rows is not None:
        lo, hi = wl.ignored_rows
        y[lo:min(hi, wl.n)] = IGNORE_INDEX
    return y


def make_inputs(wl: Workload, threads: Optional[int] = None):
    """Return (H, W, labels) as CPU torch tensors in the workload dtype (labels int64)."""
    h = _normal_rows(1000 + wl.seed, wl.n, wl.d, 1.0, threads)
    w = _normal_rows(2000 + wl.seed, wl.v, wl.d, wl.sigma_w, threads)
    y = make_labels(wl)
    ht = torch.from_numpy(h).to(wl.torch_dtype)
    del h
    wt = torch.from_numpy(w).to(wl.torch_dtype)
    del w
    return ht.contiguous(), wt.contiguous(), torch.from_numpy(y)


def make_logits(wl: Workload, sigma: Optional[float] = None, threads: Optional[int] = None):
    """Return (Z [n, v], labels) for cross-entropy on materialised logits.

    Z ~ N(0, sigma^2) in the workload dtype; the default sigma is
    sigma_w * sqrt(d), the spread of W.h for the workload's own H and W draws
    (each logit is a sum of d products of N(0, 1) and N(0, sigma_w^2) values).
    Labels are the workload's labels.  Seeds 4000 + k.
    """
    if sigma is None:
        sigma = wl.sigma_w * float(np.sqrt(wl.d))
    z = _normal_rows(4000 + wl.seed, wl.n, wl.v, sigma, threads)
    zt = torch.from_numpy(z).to(wl.torch_dtype)
    del z
    return zt.contiguous(), torch.from_numpy(make_labels(wl))


def quantize_rows_e4m3(x: torch.Tensor):
    """(codes uint8 [rows, cols], scales fp32 [rows]) of a float tensor: each row
    divided by max|row| / 448 (the largest e4m3 value; 1 for an all-zero row) and
    rounded to e4m3 by torch's round-to-nearest-even conversion."""
    x = x.float()
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x / scale[:, None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).contiguous(), scale.contiguous()


def make_inputs_fp8(wl: Workload, threads: Optional[int] = None):
    """(H codes, H scales, W codes, W scales, labels): the workload's H and W
    (float32 draws, seeds as make_inputs) quantised row by row to e4m3."""
    h = torch.from_numpy(_normal_rows(1000 + wl.seed, wl.n, wl.d, 1.0, threads))
    hq, hs = quantize_rows_e4m3(h)
    del h
    w = torch.from_numpy(_normal_rows(2000 + wl.seed, wl.v, wl.d, wl.sigma_w, threads))
    wq, ws = quantize_rows_e4m3(w)
    del w
    return hq, hs, wq, ws, torch.from_numpy(make_labels(wl))


def logits_bytes_avoided(n: int, v: int, elem_bytes: int = 4) -> int:
    """Size of the full [n, v] logits tensor that the fused path never allocates.

    The blog page's logits-memory formula (section "The 128k Vocabulary
    Explosion"): batch x sequence x vocabulary x sizeof(float32).
    """
    return int(n) * int(v) * int(elem_bytes)
