"""Planted mistakes: the oracle's pins must catch each one.

Every case below is one plausible error in one oracle function: a flipped
sign, a dropped term or factor, a wrong index or offset, a reversed operand,
a wrong normaliser or format constant.  For each case, the oracle, its pins
and the input generators are copied to a temporary directory, the one change
is written into the copy, and ``tests/test_oracle_pins.py`` runs against the
copy in a child process.  The pins must fail.  The unmutated copy must pass,
so a failure is the mutation's doing.  Nothing here touches the GPU or the
HIP library.
"""
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]

# (name, text in oracle/flce_oracle.py, replacement, occurrences replaced: 0 = all)
MUTATIONS = [
    ("fused: one-hot added instead of subtracted",
     "        g[rows, tgt] -= 1.0                        # P - onehot",
     "        g[rows, tgt] += 1.0                        # P - onehot", 0),
    ("fused: ignored rows keep their gradient",
     "        g[~valid[r0:r1]] = 0.0                     # ignored rows carry no gradient",
     "        pass", 0),
    ("fused: dW rows reversed",
     "        dw += g.T @ hd[r0:r1]                      # dL/dW = (dL/dZ)^T H",
     "        dw += (g.T @ hd[r0:r1])[::-1]", 0),
    ("fused: dH off by a relative 1e-9",
     "        dh[r0:r1] = g @ wd                         # dL/dH = (dL/dZ) W",
     "        dh[r0:r1] = g @ wd * (1 + 1e-9)", 0),
    ("fused: softmax scaled",
     "        g = np.exp(z - lse_b[:, None])             # softmax P(z)",
     "        g = np.exp(z - lse_b[:, None]) * 1.0001", 0),
    ("mean divides by the valid count plus one",
     "        return 1.0 / n_valid if n_valid > 0 else 0.0",
     "        return 1.0 / (n_valid + 1) if n_valid > 0 else 0.0", 0),
    ("NLL sign",
     "lse_b[rows] - z[rows, tgt]",
     "lse_b[rows] + z[rows, tgt]", 0),
    ("LSE without the max subtracted",
     "    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
     "    return np.log(np.exp(z).sum(axis=1))", 0),
    ("backward from the LSE: one-hot added",
     "        g[rows, y[r0 + rows]] -= 1.0",
     "        g[rows, y[r0 + rows]] += 1.0", 0),
    ("backward from the LSE: upstream gradient dropped",
     "    scale = float(grad_out) * reduction_scale(int(valid.sum()), reduction)",
     "    scale = reduction_scale(int(valid.sum()), reduction)", 1),
    ("CE on logits: one-hot in the next column",
     "    g[rows, y[rows]] -= 1.0",
     "    g[rows, (y[rows] + 1) % v] -= 1.0", 0),
    ("shards: target logit taken from the neighbouring column",
     "    zy_part[here] = z[here, local[here]]",
     "    zy_part[here] = z[here, local[here] - 1]", 0),
    ("shard merge: target logits combined by max instead of sum",
     "    zy = zp.sum(axis=0)",
     "    zy = zp.max(axis=0)", 0),
    ("shard backward: label offset by one",
     "    g[here, local[here]] -= 1.0",
     "    g[here, (local[here] + 1) % v_shard] -= 1.0", 0),
    ("e4m3: exponent bias 8",
     "np.exp2(e.astype(np.float64) - 7.0)",
     "np.exp2(e.astype(np.float64) - 8.0)", 0),
    ("e4m3: subnormal step 2^-7",
     "m / 8.0 * 2.0 ** -6",
     "m / 8.0 * 2.0 ** -7", 0),
    ("fp8 forward: H scale dropped",
     "    h = decode_e4m3(codes(h_q)) * _as_f64(h_scale)[:, None]\n"
     "    w = decode_e4m3(codes(w_q)) * _as_f64(w_scale)[:, None]\n"
     "    return flce_forward(",
     "    h = decode_e4m3(codes(h_q))\n"
     "    w = decode_e4m3(codes(w_q)) * _as_f64(w_scale)[:, None]\n"
     "    return flce_forward(", 0),
    ("fp8 backward: upstream gradient dropped",
     "    return flce_backward_from_lse(h, w, labels, lse, grad_out=grad_out,",
     "    return flce_backward_from_lse(h, w, labels, lse, grad_out=1.0,", 0),
]


def _tree(tmp: pathlib.Path) -> pathlib.Path:
    """A copy of what the pins need: the oracle, the tests and the input generators."""
    skip = shutil.ignore_patterns("__pycache__", "*.so", "*.pyc")
    for name in ("oracle", "tests", "workloads"):
        shutil.copytree(ROOT / name, tmp / name, ignore=skip)
    return tmp


def _pins(tmp: pathlib.Path) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"],
        cwd=tmp, env=env, capture_output=True, text=True, timeout=900)


def _case(base: pathlib.Path, idx: int):
    """Run the pins on copy `idx` (-1: unmutated); return the completed process."""
    tmp = _tree(base / f"case{idx + 1}")
    if idx >= 0:
        _, old, new, count = MUTATIONS[idx]
        src = tmp / "oracle" / "flce_oracle.py"
        text = src.read_text()
        if old not in text:
            raise AssertionError(f"mutation target not found: {old!r}")
        src.write_text(text.replace(old, new, count if count else -1))
    return _pins(tmp)


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every case's child run, four at a time (each is a separate pytest process)."""
    from concurrent.futures import ThreadPoolExecutor
    base = tmp_path_factory.mktemp("oracle_mutations")
    idx = list(range(-1, len(MUTATIONS)))
    with ThreadPoolExecutor(4) as ex:
        runs = list(ex.map(lambda i: _case(base, i), idx))
    return dict(zip(idx, runs))


def test_unmutated_copy_passes(outcomes):
    r = outcomes[-1]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("idx", range(len(MUTATIONS)), ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(outcomes, idx):
    r = outcomes[idx]
    assert r.returncode != 0, f"the pins did not catch: {MUTATIONS[idx][0]}\n{r.stdout[-1500:]}"
