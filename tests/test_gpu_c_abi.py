"""The C ABI from a plain C program (tests/c_abi/flce_c_check.c, built by
__graft_entry__.build() with the host C compiler; no Python or torch in it):
its flce_fwd_bwd and flce_fwd results on the null stream against the oracle,
and an argument error.  The program's inputs come from a 32-bit linear
congruential generator with values k / 64 that are exact in fp32; the same
draws are rebuilt here."""
import os
import subprocess

import numpy as np
import pytest

from oracle import flce_forward_backward

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "flce_c_check")
N, D, V = 24, 16, 40


def _inputs():
    state = 12345

    def u32():
        nonlocal state
        state = (state * 1664525 + 1013904223) & 0xFFFFFFFF
        return state

    def value():
        return float(((u32() >> 16) % 129) - 64) / 64.0

    h = np.array([value() for _ in range(N * D)], dtype=np.float64).reshape(N, D)
    w = np.array([value() * 0.5 for _ in range(V * D)], dtype=np.float64).reshape(V, D)
    y = np.array([-100 if i % 5 == 4 else u32() % V for i in range(N)], dtype=np.int64)
    return h, w, y


def test_plain_c_program_matches_the_oracle():
    assert os.path.exists(BIN), f"{BIN} is not built; run __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        name, *vals = line.split()
        out[name] = vals
    assert [int(x) for x in out["status"]] == [0, 0, -1]          # OK, OK, FLCE_ERR_INVALID_ARG
    assert out["error"], "flce_strerror gave no text"
    arr = {k: np.array([float(x) for x in v]) for k, v in out.items() if k not in ("status", "error")}
    h, w, y = _inputs()
    loss, lse, dh, dw = flce_forward_backward(h, w, y)
    assert abs(arr["loss"][0] - loss) <= 1e-5 * abs(loss)
    assert np.max(np.abs(arr["lse"] - lse) / np.abs(lse)) <= 1e-5
    assert np.max(np.abs(arr["dh"].reshape(N, D) - dh)) <= 1e-4 * np.max(np.abs(dh))
    assert np.max(np.abs(arr["dw"].reshape(V, D) - dw)) <= 1e-4 * np.max(np.abs(dw))
    # the forward-only call gives bitwise the fused call's loss and LSE
    assert np.array_equal(arr["loss_fwd"], arr["loss"]) and np.array_equal(arr["lse_fwd"], arr["lse"])
