"""Device memory of a call: the library's pool high-water mark during one fused
call equals the plan's workspace (the pool keeps one allocation per call), and
stays below the fp32 [N, V] logits the method avoids; no buffer of the plan is
a whole [N, V] array.  Inputs are seeded device draws (a memory check needs no
oracle values)."""
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SLACK = 64 << 20   # pool granularity and alignment


@pytest.mark.parametrize("n,d,v", [(8192, 4096, 128256), (32768, 4096, 128256)])
def test_fused_call_peak_memory(n, d, v):
    g = torch.Generator(device=DEV).manual_seed(n)
    h = torch.randn(n, d, device=DEV, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(v, d, device=DEV, generator=g)).to(torch.bfloat16)
    y = torch.randint(0, v, (n,), device=DEV, generator=g)
    p = flce.flce_plan_info(n, d, v, flce.FLCE_BF16, 1)
    torch.cuda.synchronize()
    flce.flce_memory_high_water(reset=True)
    flce.linear_cross_entropy(h, w, y)
    torch.cuda.synchronize()
    peak = flce.flce_memory_high_water()
    logits_fp32 = n * v * 4
    say(f"[memory] {n}x{d}x{v}: peak {peak / 1e9:.3f} GB, plan {p['workspace_bytes'] / 1e9:.3f} GB, "
        f"fp32 logits {logits_fp32 / 1e9:.2f} GB")
    assert p["workspace_bytes"] <= peak <= p["workspace_bytes"] + SLACK
    assert peak < logits_fp32
    # the largest buffer, the chunk probability buffer(s), holds fewer rows than the batch
    assert p["prob_buffer_bytes"] <= (p["chunk_rows"] * (2 if p["dw_pairs"] else 1)) * p["vocab_pitch"] * 2
    assert p["chunk_rows"] * (2 if p["dw_pairs"] else 1) < n


def test_pool_keeps_the_workspace_until_trimmed():
    """The pool keeps a finished call's workspace reserved for the next call;
    flce_pool_trim gives it back after a synchronisation, and calls after the
    trim allocate again and return the same results."""
    n, d, v = 2048, 1024, 32000
    g = torch.Generator(device=DEV).manual_seed(5)
    h = torch.randn(n, d, device=DEV, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(v, d, device=DEV, generator=g)).to(torch.bfloat16)
    y = torch.randint(0, v, (n,), device=DEV, generator=g)
    ws = flce.flce_plan_info(n, d, v, flce.FLCE_BF16, 1)["workspace_bytes"]
    first = flce.linear_cross_entropy(h, w, y)
    torch.cuda.synchronize()
    held = flce.flce_memory_reserved()
    say(f"[memory] pool after a call: {held / 1e6:.1f} MB reserved (workspace {ws / 1e6:.1f} MB)")
    assert held >= ws
    flce.flce_pool_trim(0)
    trimmed = flce.flce_memory_reserved()
    say(f"[memory] after flce_pool_trim(0): {trimmed / 1e6:.1f} MB")
    assert trimmed < ws
    again = flce.linear_cross_entropy(h, w, y)
    torch.cuda.synchronize()
    assert flce.flce_memory_reserved() >= ws
    for a, b in zip(first, again):
        assert torch.equal(a, b)
