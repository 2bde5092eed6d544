"""flce_fwd_noalloc through the C ABI: the forward in the library's fixed
scratch area, with no allocation, against flce_fwd on the same inputs (loss and
every LSE bitwise equal), on two calls in a row, the second smaller than the
first; the pool and torch's allocator see no allocation; sizes beyond the area
are refused before anything runs."""
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(n, d, v, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    h = torch.randn(n, d, device=DEV, generator=g).to(dtype)
    w = (0.05 * torch.randn(v, d, device=DEV, generator=g)).to(dtype)
    y = torch.randint(0, v, (n,), device=DEV, generator=g)
    y[::17] = -100
    return h, w, y


def _pair(n, d, v, dtype, red, seed):
    h, w, y = _inputs(n, d, v, dtype, seed)
    code = flce.FLCE_BF16 if dtype == torch.bfloat16 else flce.FLCE_F32
    s = torch.cuda.current_stream()
    ref_loss, ref_lse = torch.empty(1, device=DEV), torch.empty(n, device=DEV)
    assert flce.flce_fwd(h, w, y, n, d, v, code, -100, red, ref_loss, ref_lse, s) == flce.FLCE_OK
    loss, lse = torch.full((1,), 7.0, device=DEV), torch.full((n,), 7.0, device=DEV)
    torch.cuda.synchronize()
    flce.flce_memory_high_water(reset=True)
    before = torch.cuda.memory_allocated()
    st = flce.flce_fwd_noalloc(h, w, y, n, d, v, code, -100, red, loss, lse, s)
    torch.cuda.synchronize()
    assert st == flce.FLCE_OK, flce.flce_strerror(st)
    assert flce.flce_memory_high_water() == 0, "the library's pool handed out memory"
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(loss, ref_loss) and torch.equal(lse, ref_lse)
    return float(loss.item())


def test_noalloc_matches_flce_fwd_two_calls():
    # the Llama-3 head's forward needs two launches to fit the 64 MiB area; then a smaller, fp32, sum call
    big = _pair(8192, 4096, 128256, torch.bfloat16, flce.FLCE_MEAN, 1)
    small = _pair(300, 128, 2500, torch.float32, flce.FLCE_SUM, 2)
    assert big > 0 and small > 0


def test_noalloc_refuses_sizes_beyond_the_area():
    n, d, v = 9_000_000, 16, 1000          # 8 n bytes of per-row LSE and loss alone exceed 64 MiB
    h, w, y = _inputs(n, d, v, torch.bfloat16, 3)
    loss, lse = torch.full((1,), 7.0, device=DEV), torch.full((n,), 7.0, device=DEV)
    st = flce.flce_fwd_noalloc(h, w, y, n, d, v, flce.FLCE_BF16, -100, flce.FLCE_MEAN, loss, lse,
                               torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == flce.FLCE_ERR_SCRATCH and "scratch" in flce.flce_strerror(st)
    assert bool((loss == 7.0).all()) and bool((lse == 7.0).all())
