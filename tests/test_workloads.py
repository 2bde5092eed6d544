"""Host-side checks of the seeded input recipes and the memory arithmetic."""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from workloads import CONFIGS, IGNORE_INDEX, Workload, logits_bytes_avoided, make_inputs, make_labels

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_logits_memory_matches_printed_sizes():
    cases = json.load(open(os.path.join(GOLDEN, "logits_memory.json")))["cases"]
    for c in cases:
        b = logits_bytes_avoided(c["tokens"], c["vocab"])
        assert round(b / 1e9, c["printed_digits"]) == pytest.approx(c["printed_gb"])


def test_config_shapes():
    assert CONFIGS["llama3_8b_head"].n == 8192 and CONFIGS["llama3_8b_head"].v == 128256
    assert CONFIGS["qwen2_head"].v == 151936 and CONFIGS["qwen2_head"].d == 3584
    assert CONFIGS["long_context"].reduction == "sum"
    assert CONFIGS["tiny_f32"].dtype == "f32"


@pytest.mark.parametrize("name", list(CONFIGS))
def test_label_recipe(name):
    wl = CONFIGS[name]
    y = make_labels(wl)
    assert y.dtype == np.int64 and y.shape == (wl.n,)
    ign = y == IGNORE_INDEX
    expect = int(round(wl.ignore_frac * wl.n))
    if wl.ignored_rows is not None:
        lo, hi = wl.ignored_rows
        assert ign[lo:hi].all()
        expect_total = expect + (hi - lo)
        assert ign.sum() == expect_total
    else:
        assert ign.sum() == expect
    assert ((y[~ign] >= 0) & (y[~ign] < wl.v)).all()
    assert np.array_equal(y, make_labels(wl))            # seeded


def test_zipf_head():
    p = workloads.zipf_probabilities(151936, 1.1)
    assert p[0] == pytest.approx(0.132, abs=2e-3)
    assert p[:10].sum() == pytest.approx(0.355, abs=3e-3)
    y = make_labels(CONFIGS["qwen2_head"])
    frac0 = np.mean(y[y >= 0] == 0)
    assert 0.11 < frac0 < 0.155


def test_inputs_small_and_deterministic():
    wl = Workload("t", 300, 40, 70, "bf16", 0.02, "uniform", 0.1, "mean", seed=9)
    h1, w1, y1 = make_inputs(wl, threads=1)
    h2, w2, y2 = make_inputs(wl, threads=4)
    assert h1.dtype == torch.bfloat16 and w1.shape == (70, 40)
    assert torch.equal(h1, h2) and torch.equal(w1, w2) and torch.equal(y1, y2)
    assert abs(float(w1.float().std()) - 0.02) < 0.002


def test_block_draw_independent_of_threads():
    a = workloads._normal_rows(5, 9000, 3, 1.0, threads=1)
    b = workloads._normal_rows(5, 9000, 3, 1.0, threads=3)
    assert np.array_equal(a, b)


def test_logits_draw_deterministic_and_spread():
    from workloads import make_logits
    wl = Workload("z", 300, 4096, 5000, "f32", 0.02, "uniform", 0.1, "mean", seed=7)
    z1, y1 = make_logits(wl, threads=1)
    z2, y2 = make_logits(wl, threads=4)
    assert z1.shape == (300, 5000) and z1.dtype == torch.float32
    assert torch.equal(z1, z2) and torch.equal(y1, y2)
    assert torch.equal(y1, torch.from_numpy(make_labels(wl)))
    # default spread sigma_w * sqrt(d) = 1.28
    assert abs(float(z1.double().std()) - 1.28) < 0.01
