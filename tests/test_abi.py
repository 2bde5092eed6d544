"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, plans chunks as documented and rejects bad arguments before touching
the device."""
import ctypes
import glob
import os
import re

import pytest

import linear_cross_entropy_bwd_amd as flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(flce_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    L = flce.lib()
    names = _declared()
    assert {"flce_fwd_bwd", "flce_fwd", "flce_workspace_bytes", "flce_strerror"} <= names
    for name in sorted(names):
        assert hasattr(L, name), f"{name} declared in include/ but not exported"
    assert set(flce.EXPORTED) <= names


def test_strerror():
    for code in (0, -1, -2, -3, -4):
        assert isinstance(flce.flce_strerror(code), str) and flce.flce_strerror(code)
    assert flce.flce_strerror(-99) == "unknown status"


@pytest.mark.parametrize("dtype", [flce.FLCE_BF16, flce.FLCE_F32])
@pytest.mark.parametrize("shape", [(256, 512, 4096), (8192, 4096, 128256), (4096, 3584, 151936),
                                   (32768, 4096, 128256), (16384, 4096, 32000), (37, 72, 1001), (1, 8, 3)])
def test_plan_invariants(dtype, shape):
    n, d, v = shape
    p = flce.flce_plan_info(n, d, v, dtype, 1)
    c = p["chunk_rows"]
    assert 1 <= c <= n
    assert p["num_chunks"] == -(-n // c)
    if n >= 32:
        assert c < n                                  # never a whole [n, v] buffer
        assert p["prob_buffer_bytes"] < n * v * 4     # below the fp32 logits it replaces
    assert p["vocab_pitch"] >= v and p["vocab_pitch"] % 256 == 0
    assert p["workspace_bytes"] == flce.flce_workspace_bytes(n, d, v, dtype, 1)
    assert p["workspace_bytes"] >= p["prob_buffer_bytes"]
    # two chunk buffers (one dW launch per chunk pair) exactly when a bf16 plan has four or more chunks
    assert p["dw_pairs"] == int(dtype == flce.FLCE_BF16 and p["num_chunks"] >= 4)
    fwd = flce.flce_plan_info(n, d, v, dtype, 0)
    assert fwd["prob_buffer_bytes"] == 0 and fwd["dw_pairs"] == 0
    assert fwd["workspace_bytes"] <= p["workspace_bytes"]
    # the per-row factor of the one-pass backward: bf16 with a pitch of at least 2 d;
    # its bf16 copy of H (one per chunk buffer) is what sets the one-pass workspace
    # above the recompute backward's
    fold = int(dtype == flce.FLCE_BF16 and p["vocab_pitch"] >= 2 * d)
    assert p["folded_factor"] == fold
    rec = flce.flce_plan_info(n, d, v, dtype, 2)
    assert rec["folded_factor"] == 0 and fwd["folded_factor"] == 0
    assert (rec["chunk_rows"], rec["dw_pairs"], rec["prob_buffer_bytes"]) == (c, p["dw_pairs"], p["prob_buffer_bytes"])
    hs = c * d * 2 * (2 if p["dw_pairs"] else 1)
    assert fold * hs <= p["workspace_bytes"] - rec["workspace_bytes"] <= fold * (hs + 4 * 256 + 16 * c + 3 * 256)
    assert rec["workspace_bytes"] == flce.flce_workspace_bytes(n, d, v, dtype, 2)


def test_plan_env_overrides(monkeypatch):
    monkeypatch.setenv("FLCE_CHUNK_ROWS", "96")
    assert flce.flce_plan_info(1000, 64, 500, flce.FLCE_F32, 1)["chunk_rows"] == 96
    monkeypatch.delenv("FLCE_CHUNK_ROWS")
    monkeypatch.setenv("FLCE_WORKSPACE_CAP_BYTES", str(64 * 1024 * 1024))
    p = flce.flce_plan_info(8192, 4096, 128256, flce.FLCE_BF16, 1)
    assert p["chunk_rows"] * p["vocab_pitch"] * 2 <= 64 * 1024 * 1024     # the cap bounds one chunk's buffer
    assert p["dw_pairs"] == 1 and p["prob_buffer_bytes"] == 2 * p["chunk_rows"] * p["vocab_pitch"] * 2
    monkeypatch.delenv("FLCE_WORKSPACE_CAP_BYTES")
    assert flce.flce_plan_info(8192, 4096, 128256, flce.FLCE_BF16, 1)["folded_factor"] == 1
    monkeypatch.setenv("FLCE_INPLACE_GRAD", "1")
    assert flce.flce_plan_info(8192, 4096, 128256, flce.FLCE_BF16, 1)["folded_factor"] == 0


def test_invalid_sizes():
    assert flce.flce_workspace_bytes(0, 8, 8, flce.FLCE_F32, 1) == 0
    assert flce.flce_workspace_bytes(8, -1, 8, flce.FLCE_F32, 1) == 0
    assert flce.flce_workspace_bytes(8, 8, 8, 7, 1) == 0
    with pytest.raises(flce.FlceError):
        flce.flce_plan_info(8, 8, 0, flce.FLCE_F32, 1)


def test_dimension_limits():
    # row strides stay below 2^24 elements: d <= 2^24, v <= 2^24 - 256
    big = 1 << 24
    flce.flce_plan_info(8, big, 8, flce.FLCE_BF16, 1)
    flce.flce_plan_info(8, 8, big - 256, flce.FLCE_BF16, 1)
    for d, v in ((big + 1, 8), (8, big - 255)):
        with pytest.raises(flce.FlceError):
            flce.flce_plan_info(8, d, v, flce.FLCE_BF16, 1)
        assert flce.flce_workspace_bytes(8, d, v, flce.FLCE_BF16, 1) == 0


def test_argument_errors_before_any_device_work():
    # All of these fail validation before the library makes a HIP call.
    A = 1 << 20  # fake, 16-byte aligned addresses: never dereferenced
    ok = dict(h=A, w=A, labels=A, n=4, d=8, v=16, dtype=flce.FLCE_F32, ignore_index=-100,
              reduction=flce.FLCE_MEAN, loss_out=A, lse_out=None, dh_out=A, dw_out=A, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return flce.flce_fwd_bwd(**a)

    assert call(h=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(labels=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(loss_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(dh_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(n=0) == flce.FLCE_ERR_INVALID_ARG
    assert call(d=-3) == flce.FLCE_ERR_INVALID_ARG
    assert call(dtype=5) == flce.FLCE_ERR_INVALID_ARG
    assert call(reduction=9) == flce.FLCE_ERR_INVALID_ARG
    assert call(h=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert call(dw_out=A + 8) == flce.FLCE_ERR_ALIGNMENT
    assert call(d=6) == flce.FLCE_ERR_ALIGNMENT           # 24-byte fp32 rows
    assert call(dtype=flce.FLCE_BF16, d=12) == flce.FLCE_ERR_ALIGNMENT
    assert call(labels=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert flce.flce_fwd(None, A, A, 4, 8, 16, flce.FLCE_F32, -100, 0, A, None, None) == flce.FLCE_ERR_INVALID_ARG


def test_bwd_argument_errors_before_any_device_work():
    A = 1 << 20  # fake, 16-byte aligned addresses: never dereferenced
    ok = dict(h=A, w=A, labels=A, lse=A, grad_out=None, n=4, d=8, v=16, dtype=flce.FLCE_F32, ignore_index=-100,
              reduction=flce.FLCE_MEAN, dh_out=A, dw_out=A, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return flce.flce_bwd(**a)

    assert call(lse=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(h=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(dh_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(dw_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(v=0) == flce.FLCE_ERR_INVALID_ARG
    assert call(reduction=7) == flce.FLCE_ERR_INVALID_ARG
    assert call(lse=A + 2) == flce.FLCE_ERR_ALIGNMENT
    assert call(grad_out=A + 2) == flce.FLCE_ERR_ALIGNMENT
    assert call(dh_out=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert call(d=6) == flce.FLCE_ERR_ALIGNMENT


def test_ce_logits_argument_errors_before_any_device_work():
    A = 1 << 20
    ok = dict(logits=A, labels=A, n=4, v=16, dtype=flce.FLCE_BF16, ignore_index=-100, reduction=flce.FLCE_MEAN,
              lse_in=None, grad_scale=None, loss_out=A, lse_out=None, grad_out=None, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return flce.flce_ce_logits(**a)

    assert call(logits=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(labels=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(n=0) == flce.FLCE_ERR_INVALID_ARG
    assert call(v=-1) == flce.FLCE_ERR_INVALID_ARG
    assert call(dtype=3) == flce.FLCE_ERR_INVALID_ARG
    assert call(loss_out=None) == flce.FLCE_ERR_INVALID_ARG              # statistics without a loss output
    assert call(lse_in=A, loss_out=None) == flce.FLCE_ERR_INVALID_ARG    # a backward without a gradient output
    assert call(logits=A + 1) == flce.FLCE_ERR_ALIGNMENT
    assert call(grad_out=A + 1) == flce.FLCE_ERR_ALIGNMENT
    assert call(dtype=flce.FLCE_F32, logits=A + 2) == flce.FLCE_ERR_ALIGNMENT
    assert call(labels=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert call(lse_out=A + 2) == flce.FLCE_ERR_ALIGNMENT


def test_shard_argument_errors_before_any_device_work():
    A = 1 << 20
    fw = dict(h=A, w_shard=A, labels=A, n=4, d=64, v_shard=300, v_first=1000, dtype=flce.FLCE_BF16,
              ignore_index=-100, lse_part_out=A, zy_part_out=A, stream=None)

    def fwd(**kw):
        a = dict(fw)
        a.update(kw)
        return flce.flce_fwd_shard(**a)

    assert fwd(lse_part_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert fwd(zy_part_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert fwd(v_first=-1) == flce.FLCE_ERR_INVALID_ARG
    assert fwd(v_shard=0) == flce.FLCE_ERR_INVALID_ARG
    assert fwd(ignore_index=-(1 << 63)) == flce.FLCE_ERR_INVALID_ARG     # shifted ignore value would wrap
    assert fwd(w_shard=A + 8) == flce.FLCE_ERR_ALIGNMENT
    assert fwd(zy_part_out=A + 2) == flce.FLCE_ERR_ALIGNMENT

    mg = dict(lse_parts=A, zy_parts=A, num_shards=3, labels=A, n=4, ignore_index=-100, reduction=flce.FLCE_MEAN,
              loss_out=A, lse_out=None, stream=None)

    def merge(**kw):
        a = dict(mg)
        a.update(kw)
        return flce.flce_merge_shards(**a)

    assert merge(num_shards=0) == flce.FLCE_ERR_INVALID_ARG
    assert merge(loss_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert merge(reduction=5) == flce.FLCE_ERR_INVALID_ARG
    assert merge(labels=A + 4) == flce.FLCE_ERR_ALIGNMENT

    bw = dict(h=A, w_shard=A, labels=A, lse=A, grad_out=None, n=4, d=64, v_shard=300, v_first=0,
              dtype=flce.FLCE_BF16, ignore_index=-100, reduction=flce.FLCE_SUM, dh_part_out=A, dw_shard_out=A,
              stream=None)

    def bwd(**kw):
        a = dict(bw)
        a.update(kw)
        return flce.flce_bwd_shard(**a)

    assert bwd(lse=None) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(dh_part_out=None) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(v_first=-5) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(dh_part_out=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert bwd(grad_out=A + 2) == flce.FLCE_ERR_ALIGNMENT

    assert flce.flce_sum_parts(A, 0, 10, flce.FLCE_BF16, A, None) == flce.FLCE_ERR_INVALID_ARG
    assert flce.flce_sum_parts(None, 2, 10, flce.FLCE_BF16, A, None) == flce.FLCE_ERR_INVALID_ARG
    assert flce.flce_sum_parts(A, 2, 10, 7, A, None) == flce.FLCE_ERR_INVALID_ARG
    assert flce.flce_sum_parts(A, 2, 10, flce.FLCE_F32, A + 2, None) == flce.FLCE_ERR_ALIGNMENT


def test_fp8_argument_errors_before_any_device_work():
    A = 1 << 20
    ok = dict(h_q=A, h_scale=A, w_q=A, w_scale=A, labels=A, n=4, d=64, v=300, ignore_index=-100,
              reduction=flce.FLCE_MEAN, loss_out=A, lse_out=None, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return flce.flce_fwd_fp8(**a)

    for k in ("h_q", "h_scale", "w_q", "w_scale", "labels", "loss_out"):
        assert call(**{k: None}) == flce.FLCE_ERR_INVALID_ARG, k
    assert call(n=0) == flce.FLCE_ERR_INVALID_ARG
    assert call(reduction=9) == flce.FLCE_ERR_INVALID_ARG
    assert call(d=72) == flce.FLCE_ERR_ALIGNMENT            # rows must be whole 16-byte vectors
    assert call(h_q=A + 8) == flce.FLCE_ERR_ALIGNMENT
    assert call(w_scale=A + 4) == flce.FLCE_ERR_ALIGNMENT
    assert call(h_scale=A + 2) == flce.FLCE_ERR_ALIGNMENT
    assert call(d=(1 << 25) + 32) == flce.FLCE_ERR_INVALID_ARG   # beyond the engine's row length


def test_fp8_backward_argument_errors_before_any_device_work():
    A = 1 << 20
    ok = dict(h_q=A, h_scale=A, w_q=A, w_scale=A, labels=A, lse=A, grad_out=None, n=4, d=64, v=300,
              ignore_index=-100, reduction=flce.FLCE_MEAN, dh_out=A, dw_out=A, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return flce.flce_bwd_fp8(**a)

    for k in ("h_q", "h_scale", "w_q", "w_scale", "labels", "lse", "dh_out", "dw_out"):
        assert call(**{k: None}) == flce.FLCE_ERR_INVALID_ARG, k
    assert call(v=0) == flce.FLCE_ERR_INVALID_ARG
    assert call(d=40) == flce.FLCE_ERR_ALIGNMENT
    assert call(dw_out=A + 8) == flce.FLCE_ERR_ALIGNMENT
    assert call(grad_out=A + 2) == flce.FLCE_ERR_ALIGNMENT


def test_vocab_shard_bounds():
    assert flce.vocab_shard_bounds(128256, 8)[0] == (0, 15872)
    for v, q in [(128256, 8), (1000, 3), (5, 5), (1 << 20, 7), (300, 2)]:
        b = flce.vocab_shard_bounds(v, q)
        assert len(b) == q and b[0][0] == 0 and b[-1][1] == v
        assert all(x < y for x, y in b) and all(b[i][1] == b[i + 1][0] for i in range(q - 1))


def test_no_cpu_fallback(monkeypatch, tmp_path):
    """Without the built library the binding raises instead of computing anything."""
    monkeypatch.setattr(flce, "_lib", None)
    monkeypatch.setattr(flce, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        flce.lib()


def test_fp8_wrappers_reject_host_tensors():
    """The FP8 wrappers check their tensors before anything reaches the library."""
    import torch
    hq = torch.zeros(4, 16, dtype=torch.uint8)
    wq = torch.zeros(8, 16, dtype=torch.uint8)
    hs, ws = torch.ones(4), torch.ones(8)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_forward_fp8(hq, hs, wq, ws, y)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy_backward_fp8(hq, hs, wq, ws, y, torch.zeros(4))


@pytest.mark.parametrize("dtype", [flce.FLCE_BF16, flce.FLCE_F32])
@pytest.mark.parametrize("shape", [(256, 512, 4096), (8192, 4096, 128256), (4096, 3584, 151936),
                                   (32768, 4096, 128256), (16384, 4096, 32000), (37, 72, 1001), (300, 128, 2500)])
def test_lowmem_plan_invariants(dtype, shape):
    n, d, v = shape
    p = flce.flce_lowmem_plan_info(n, d, v, dtype)
    vb, q = p["slice_cols"], p["num_slices"]
    assert q == -(-v // vb) and (vb % 256 == 0 or q == 1)
    assert q >= 2 or p["slice_chunk_rows"] < n or n < 32      # no buffer spans [n, v]
    elem = 2 if dtype == flce.FLCE_BF16 else 4
    assert p["slice_chunk_rows"] * vb * elem <= max(p["buffer_budget_bytes"], p["slice_chunk_rows"] * 256 * elem)
    assert p["workspace_bytes"] == flce.flce_workspace_bytes_lowmem(n, d, v, dtype)
    assert p["workspace_bytes"] < n * v * 4
    if (n, d, v) == (8192, 4096, 128256):
        # the Llama-3 head: the low-memory path holds under a fifth of the fp32 logits it avoids
        assert p["workspace_bytes"] <= 0.2 * n * v * 4
        assert p["slice_chunks"] == 1                          # each slice's dW is one reduction over all tokens


def test_lowmem_budget_override(monkeypatch):
    monkeypatch.setenv("FLCE_LOWMEM_BUFFER_BYTES", str(600 * 1000))
    p = flce.flce_lowmem_plan_info(300, 128, 2500, flce.FLCE_BF16)
    assert p["slice_cols"] == 768 and p["num_slices"] == 4          # 600 kB / (300 rows x 2 B) -> 3 x 256 columns
    assert flce.flce_workspace_bytes_lowmem(0, 8, 8, flce.FLCE_BF16) == 0


def test_dh_split_partials_stay_below_the_chunk_buffer():
    for shape, dtype in [((256, 512, 4096), flce.FLCE_F32), ((4096, 3584, 151936), flce.FLCE_BF16),
                         ((37, 72, 1001), flce.FLCE_F32), ((8192, 4096, 128256), flce.FLCE_BF16)]:
        n, d, v = shape
        p = flce.flce_plan_info(n, d, v, dtype, 1)
        if p["dh_splits"] > 1:
            assert p["dh_splits"] * p["chunk_rows"] * d * 4 <= max(p["prob_buffer_bytes"], p["chunk_rows"] * d * 4)
        assert p["workspace_bytes"] < n * v * 4 or n < 256   # tiny shapes: 16-row chunk rounding and alignment


def test_row_count_limit():
    """n_valid is counted in 32 bits, so more than 2^31 - 1 token rows is an argument error."""
    assert flce.flce_workspace_bytes(2**31 - 1, 16, 64, flce.FLCE_BF16, 0) > 0
    assert flce.flce_workspace_bytes(2**31, 16, 64, flce.FLCE_BF16, 0) == 0
    assert flce.flce_workspace_bytes(2**31, 16, 64, flce.FLCE_BF16, 1) == 0
    assert flce.flce_workspace_bytes_lowmem(2**31, 16, 64, flce.FLCE_BF16) == 0
