"""How the error of dW behaves as the number of token chunks grows.

Across chunks the fused call keeps dW as an exact fp32 sum, its upper 16 bits
in dw_out and its lower 16 bits in the workspace; only the last chunk rounds
it to bf16.  This measures dW's error against the full fp64 oracle for 2, 8,
32 and 64 chunks (FLCE_CHUNK_ROWS 4096, 1024, 256, 128 on 8192 x 1024 x 32000;
plans of four or more chunks pair them, so 64 chunks are 32 dW launches over
the running sum), next to the low-memory path, whose dW rows are single fp32
reductions over all tokens.  Every count must stay within the 2e-2 bound.
Measured: the error does not grow with the count (the Frobenius error is the
same at 2 and 64 chunks; 64 chunks move 0.02% of the entries by one bf16
step, the fp32 rounding of the partial sums); it is set by G's bf16 rounding."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_bwd_amd as flce
from oracle import flce_forward_backward
from workloads import Workload, make_inputs

from gpu_helpers import rel_max, say, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
WL = Workload("dw_chunks", 8192, 1024, 32000, "bf16", 0.02, "uniform", 0.05, "mean", seed=61)
_REF = {}


def _ref():
    if not _REF:
        h, w, y = make_inputs(WL)
        _REF["inputs"] = (h, w, y)
        _REF["oracle"] = flce_forward_backward(h, w, y)
    return _REF["inputs"], _REF["oracle"]


@pytest.mark.parametrize("chunk,chunks", [("4096", 2), ("1024", 8), ("256", 32), ("128", 64), ("lowmem", 1)])
def test_dw_error_against_chunk_count(monkeypatch, chunk, chunks):
    (h, w, y), (rl, rlse, rdh, rdw) = _ref()
    hd, wd, yd = h.cuda(), w.cuda(), y.cuda()
    if chunk == "lowmem":
        out = flce.linear_cross_entropy_lowmem(hd, wd, yd)
    else:
        monkeypatch.setenv("FLCE_CHUNK_ROWS", chunk)
        assert flce.flce_plan_info(WL.n, WL.d, WL.v, flce.FLCE_BF16, 1)["num_chunks"] == chunks
        out = flce.linear_cross_entropy(hd, wd, yd)
    torch.cuda.synchronize()
    loss, lse, dh, dw = out
    gdw = to_f64(dw)
    e_dw = rel_max(gdw, rdw)
    e_dh = rel_max(to_f64(dh), rdh)
    # The max-abs norm saturates near one bf16 step of the largest entries whatever the
    # accumulation does, so two finer measures go with it: the relative Frobenius error,
    # and the share of entries that differ from the correctly rounded exact value.
    exact16 = torch.from_numpy(rdw).to(torch.bfloat16).double().numpy()
    floor_max = rel_max(exact16, rdw)
    frob = float(np.linalg.norm(gdw - rdw) / np.linalg.norm(rdw))
    frob_floor = float(np.linalg.norm(exact16 - rdw) / np.linalg.norm(rdw))
    differ = float(np.mean(gdw != exact16))
    # and the entries that differ from the two-chunk result, by how much
    _REF.setdefault("first", gdw)
    moved = gdw != _REF["first"]
    say(f"  entries differing from the first chunking measured: {int(moved.sum())} of {gdw.size}, "
        f"largest difference {float(np.max(np.abs(gdw - _REF['first']))):.3e}")
    say(f"[dW chunks] {chunk} ({chunks} chunks): dW max-abs {e_dw:.3e} (rounding alone {floor_max:.3e}), "
        f"Frobenius {frob:.3e} (rounding alone {frob_floor:.3e}), entries off the rounded exact value "
        f"{100 * differ:.2f}%; dH {e_dh:.3e}; loss rel {abs(float(loss.item()) - rl) / abs(rl):.2e}")
    assert e_dw <= 2e-2 and e_dh <= 2e-2
    assert frob <= 3 * frob_floor
