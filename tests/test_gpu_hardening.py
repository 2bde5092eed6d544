"""Failure handling and out-of-bounds writes.

* Every call that allocates a workspace returns FLCE_ERR_OOM, enqueues nothing
  and writes nothing when the allocation fails (forced from the host through the
  FLCE_TEST_ALLOC_LIMIT_BYTES hook, so no kernel ever sees the condition), and a
  normal call afterwards is unaffected.
* Outputs handed to the library sit inside larger allocations filled with a
  sentinel pattern; after the call the sentinels around every output are
  unchanged, on ragged shapes and with chunked and paired plans, and the
  results inside still match the oracle.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_forward_backward
from workloads import Workload, make_inputs

from gpu_helpers import check, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD = 256                                    # sentinel elements on each side (keeps 16-byte alignment)
SENT = {torch.bfloat16: (torch.int16, 0x5A5A), torch.float32: (torch.int32, 0x5A5A5A5A)}


def guarded(shape, dtype):
    """(whole sentinel-filled buffer, contiguous view of `shape` inside it)."""
    n = int(np.prod(shape))
    raw_t, pat = SENT[dtype]
    buf = torch.empty(n + 2 * PAD, dtype=dtype, device=DEV)
    buf.view(raw_t).fill_(pat)
    return buf, buf[PAD:PAD + n].view(shape)


def intact(buf, shape):
    n = int(np.prod(shape))
    raw_t, pat = SENT[buf.dtype]
    raw = buf.view(raw_t)
    return bool((raw[:PAD] == pat).all()) and bool((raw[PAD + n:] == pat).all())


def _inputs(n, d, v, dtype, seed, ignore_frac=0.1):
    wl = Workload("guard", n, d, v, dtype, 0.1, "uniform", ignore_frac, "mean", seed=seed)
    h, w, y = make_inputs(wl, threads=4)
    return wl, h, w, y


SHAPES = [(513, 520, 2100, "bf16", None), (1, 16, 5, "bf16", None), (37, 72, 1001, "f32", None),
          (513, 520, 2100, "bf16", "128")]     # 128-row chunks: five chunks, two pairs and a lone last chunk


@pytest.mark.parametrize("n,d,v,dtype,chunk", SHAPES)
def test_fused_and_lowmem_outputs_stay_in_bounds(monkeypatch, n, d, v, dtype, chunk):
    if chunk:
        monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
    wl, h, w, y = _inputs(n, d, v, dtype, seed=51)
    tdt = wl.torch_dtype
    code = flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    ref = flce_forward_backward(h, w, y)
    s = torch.cuda.current_stream()
    for name, fn in (("flce_fwd_bwd", flce.flce_fwd_bwd), ("flce_fwd_bwd_lowmem", flce.flce_fwd_bwd_lowmem)):
        bl, loss = guarded((1,), torch.float32)
        bs, lse = guarded((n,), torch.float32)
        bh, dh = guarded((n, d), tdt)
        bw, dw = guarded((v, d), tdt)
        st = fn(hd, wd, yd, n, d, v, code, -100, flce.FLCE_MEAN, loss, lse, dh, dw, s)
        torch.cuda.synchronize()
        assert st == flce.FLCE_OK
        for b, shp, what in ((bl, (1,), "loss"), (bs, (n,), "lse"), (bh, (n, d), "dH"), (bw, (v, d), "dW")):
            assert intact(b, shp), f"{name} wrote outside {what}"
        check((float(loss.item()), to_f64(lse), to_f64(dh), to_f64(dw)), ref, tdt, f"{name} guarded")


@pytest.mark.parametrize("n,d,v,dtype,chunk", SHAPES[:3])
def test_split_and_shard_outputs_stay_in_bounds(n, d, v, dtype, chunk):
    wl, h, w, y = _inputs(n, d, v, dtype, seed=52)
    tdt = wl.torch_dtype
    code = flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    s = torch.cuda.current_stream()
    bl, loss = guarded((1,), torch.float32)
    bs, lse = guarded((n,), torch.float32)
    assert flce.flce_fwd(hd, wd, yd, n, d, v, code, -100, flce.FLCE_MEAN, loss, lse, s) == flce.FLCE_OK
    bh, dh = guarded((n, d), tdt)
    bw, dw = guarded((v, d), tdt)
    assert flce.flce_bwd(hd, wd, yd, lse, None, n, d, v, code, -100, flce.FLCE_MEAN, dh, dw, s) == flce.FLCE_OK
    torch.cuda.synchronize()
    for b, shp, what in ((bl, (1,), "loss"), (bs, (n,), "lse"), (bh, (n, d), "dH"), (bw, (v, d), "dW")):
        assert intact(b, shp), f"split path wrote outside {what}"
    # one vocabulary shard of the upper part of W
    a = v // 2
    vs = v - a
    blp, lse_p = guarded((n,), torch.float32)
    bzp, zy_p = guarded((n,), torch.float32)
    assert flce.flce_fwd_shard(hd, wd[a:], yd, n, d, vs, a, code, -100, lse_p, zy_p, s) == flce.FLCE_OK
    bdp, dh_p = guarded((n, d), torch.float32)
    bws, dw_s = guarded((vs, d), tdt)
    assert flce.flce_bwd_shard(hd, wd[a:], yd, lse, None, n, d, vs, a, code, -100, flce.FLCE_MEAN, dh_p, dw_s,
                               s) == flce.FLCE_OK
    # and the lower part of W added into the same dH sum
    bws2, dw_s2 = guarded((a, d), tdt)
    assert flce.flce_bwd_shard_accumulate(hd, wd[:a], yd, lse, None, n, d, a, 0, code, -100, flce.FLCE_MEAN, dh_p,
                                          dw_s2, s) == flce.FLCE_OK
    torch.cuda.synchronize()
    for b, shp, what in ((blp, (n,), "shard lse"), (bzp, (n,), "shard zy"), (bdp, (n, d), "shard dH part"),
                         (bws, (vs, d), "shard dW"), (bws2, (a, d), "second shard dW")):
        assert intact(b, shp), f"shard path wrote outside {what}"
    ref = flce_forward_backward(h, w, y)
    np.testing.assert_allclose(to_f64(dw_s), to_f64(dw)[a:], rtol=0, atol=2e-2 * float(np.max(np.abs(ref[3]))))
    np.testing.assert_allclose(to_f64(dw_s2), to_f64(dw)[:a], rtol=0, atol=2e-2 * float(np.max(np.abs(ref[3]))))
    # the two shards' terms summed are the whole dH
    np.testing.assert_allclose(to_f64(dh_p), ref[2], rtol=0, atol=2e-2 * float(np.max(np.abs(ref[2]))))


@pytest.mark.parametrize("n,v,dtype", [(513, 2100, "bf16"), (37, 1001, "f32"), (3, 7, "bf16")])
def test_ce_logits_outputs_stay_in_bounds(n, v, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = flce.FLCE_BF16 if dtype == "bf16" else flce.FLCE_F32
    g = torch.Generator().manual_seed(53)
    z = (3.0 * torch.randn(n, v, generator=g)).to(tdt).to(DEV)
    y = torch.randint(0, v, (n,), generator=g)
    y[::4] = -100
    yd = y.to(DEV)
    s = torch.cuda.current_stream()
    bl, loss = guarded((1,), torch.float32)
    bs, lse = guarded((n,), torch.float32)
    bg, grad = guarded((n, v), tdt)
    assert flce.flce_ce_logits(z, yd, n, v, code, -100, flce.FLCE_MEAN, None, None, loss, lse, grad,
                               s) == flce.FLCE_OK
    bg2, grad2 = guarded((n, v), tdt)
    assert flce.flce_ce_logits(z, yd, n, v, code, -100, flce.FLCE_MEAN, lse, None, None, None, grad2,
                               s) == flce.FLCE_OK
    torch.cuda.synchronize()
    for b, shp, what in ((bl, (1,), "loss"), (bs, (n,), "lse"), (bg, (n, v), "gradient"),
                         (bg2, (n, v), "gradient from the LSE")):
        assert intact(b, shp), f"flce_ce_logits wrote outside {what}"


def test_allocation_failure_returns_oom_and_writes_nothing(monkeypatch):
    n, d, v = 300, 128, 2500
    wl, h, w, y = _inputs(n, d, v, "bf16", seed=54)
    hd, wd, yd = h.to(DEV), w.to(DEV), y.to(DEV)
    s = torch.cuda.current_stream()
    B, M, OOM = flce.FLCE_BF16, flce.FLCE_MEAN, flce.FLCE_ERR_OOM
    hq = torch.zeros(n, d, dtype=torch.uint8, device=DEV)
    wq = torch.zeros(v, d, dtype=torch.uint8, device=DEV)
    hs = torch.ones(n, device=DEV)
    ws = torch.ones(v, device=DEV)
    lse0 = torch.full((n,), 1.0, device=DEV)
    z = torch.zeros(n, v, dtype=torch.bfloat16, device=DEV)
    parts = torch.zeros(2, n, device=DEV)
    outs = {"loss": torch.full((1,), 7.0, device=DEV), "lse": torch.full((n,), 7.0, device=DEV),
            "dh": torch.full((n, d), 7.0, dtype=torch.bfloat16, device=DEV),
            "dw": torch.full((v, d), 7.0, dtype=torch.bfloat16, device=DEV),
            "dhp": torch.full((n, d), 7.0, device=DEV), "g": torch.full((n, v), 7.0, dtype=torch.bfloat16, device=DEV)}
    o = outs
    calls = {
        "flce_fwd_bwd": lambda: flce.flce_fwd_bwd(hd, wd, yd, n, d, v, B, -100, M, o["loss"], o["lse"], o["dh"], o["dw"], s),
        "flce_fwd_bwd_lowmem": lambda: flce.flce_fwd_bwd_lowmem(hd, wd, yd, n, d, v, B, -100, M, o["loss"], o["lse"],
                                                                o["dh"], o["dw"], s),
        "flce_fwd": lambda: flce.flce_fwd(hd, wd, yd, n, d, v, B, -100, M, o["loss"], o["lse"], s),
        "flce_bwd": lambda: flce.flce_bwd(hd, wd, yd, lse0, None, n, d, v, B, -100, M, o["dh"], o["dw"], s),
        "flce_ce_logits": lambda: flce.flce_ce_logits(z, yd, n, v, B, -100, M, None, None, o["loss"], o["lse"], o["g"], s),
        "flce_fwd_fp8": lambda: flce.flce_fwd_fp8(hq, hs, wq, ws, yd, n, d, v, -100, M, o["loss"], o["lse"], s),
        "flce_bwd_fp8": lambda: flce.flce_bwd_fp8(hq, hs, wq, ws, yd, lse0, None, n, d, v, -100, M, o["dh"], o["dw"], s),
        "flce_fwd_shard": lambda: flce.flce_fwd_shard(hd, wd[:1000], yd, n, d, 1000, 0, B, -100, o["lse"], parts[0], s),
        "flce_merge_shards": lambda: flce.flce_merge_shards(parts, parts, 2, yd, n, -100, M, o["loss"], o["lse"], s),
        "flce_bwd_shard": lambda: flce.flce_bwd_shard(hd, wd[:1000], yd, lse0, None, n, d, 1000, 0, B, -100, M,
                                                      o["dhp"], o["dw"][:1000], s),
        "flce_bwd_shard_accumulate": lambda: flce.flce_bwd_shard_accumulate(hd, wd[:1000], yd, lse0, None, n, d, 1000,
                                                                            0, B, -100, M, o["dhp"], o["dw"][:1000], s),
    }
    torch.cuda.synchronize()
    monkeypatch.setenv("FLCE_TEST_ALLOC_LIMIT_BYTES", "1")
    for name, fn in calls.items():
        st = fn()
        assert st == OOM, f"{name} returned {st}"
        assert "allocation" in flce.flce_strerror(st)
    torch.cuda.synchronize()
    for k, t in outs.items():
        assert bool((t == 7.0).all()), f"an output ({k}) was written by a call that failed"
    monkeypatch.delenv("FLCE_TEST_ALLOC_LIMIT_BYTES")
    loss, lse, dh, dw = flce.linear_cross_entropy(hd, wd, yd)
    torch.cuda.synchronize()
    check((float(loss.item()), to_f64(lse), to_f64(dh), to_f64(dw)), flce_forward_backward(h, w, y),
          torch.bfloat16, "after the failed calls")
