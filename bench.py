"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

One step = one flce_fwd_bwd call (label scan; per chunk the target-logit
reference, the logits GEMM with the online LSE / target epilogue, the merge,
the per-row factor patch, dH and dW GEMMs; loss reduction) over the
Llama-3-8B LM-head workload: N=8192 tokens, D=4096,
V=128256, bf16, 5% ignored labels, mean reduction.  Inputs are synthetic,
seeded and resident in HBM before timing starts.  The headline `value` and
`ms_per_step` come from steps timed without any per-kernel instrumentation;
a second pass with the library's HIP-event instrumentation gives the
per-kernel split and the roofline figures.

By default the line also carries every workload (`per_config`: tokens/s,
matrix-peak fraction, extra device memory against the N V 4 bytes of logits
avoided, and parity against the fp64 oracle), the parity of the headline
workload, the low-memory path and a memory/speed sweep, the other entry
points (split forward/backward, the in-place gradient form of the fused call,
forward only, vocabulary split, FP8, cross-entropy on given logits), torch's hipBLASLt products on the same
contraction shapes for context, and the oracle's CPU baseline.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s (N=8192,D=4096,V=128256 bf16); MFMA %"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}      # MI355X dense matrix peaks
GEMM_KINDS = ("logits_lse", "dh_gemm", "dw_gemm")
COPY_BYTES = 1 << 30
HBM_PEAK_GBPS = 8000.0                               # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_llama3_8b_head_traffic.txt")
TRAFFIC_KEYS = {"logits_lse": ("logits", "engine"), "dh_gemm": ("dh", "engine"), "dw_gemm": ("dw", "engine"),
                "ce_fwd_grad": ("ce_fwd_grad", "ce")}
KERNEL_SRC = {"engine": os.path.join(ROOT, "linear_cross_entropy_bwd_amd", "csrc", "engine_mfma.hip"),
              "ce": os.path.join(ROOT, "linear_cross_entropy_bwd_amd", "csrc", "ce_logits.hip")}


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    there is none or the kernel's source changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE) or kernel not in TRAFFIC_KEYS:
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    key, src = TRAFFIC_KEYS[kernel]
    digest = hashlib.sha256(open(KERNEL_SRC[src], "rb").read()).hexdigest()
    if kv.get(f"{src}_sha256") != digest:
        return None
    try:
        return float(kv[f"{key}_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(wl, h, w, y, rows: int):
    """The fp64 oracle, as it stands, on the first `rows` tokens of the same workload."""
    import numpy as np

    from oracle import flce_forward_backward
    cores = len(os.sched_getaffinity(0))
    hs, ys = h[:rows], y[:rows]
    t0 = time.perf_counter()
    flce_forward_backward(hs, w, ys, reduction=wl.reduction)
    dt = time.perf_counter() - t0
    del np
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of {wl.n} tokens of {wl.name} (full D={wl.d}, V={wl.v}), fp64 numpy, "
                      f"{dt:.1f} s incl. fp64 conversion"}


def median(xs):
    t = sorted(xs)
    return t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])


def time_steps(torch, fn, stream, steps, warmup):
    """Per-step milliseconds of `fn` (HIP events on `stream` between the steps), after
    `warmup` untimed calls; no instrumentation of the library is on."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)], ev[0].elapsed_time(ev[-1])


def sample_rows(n, chunk, y, rng):
    """Token rows the parity check compares: the first and last row, both sides of every
    chunk boundary, 16 random rows and up to 4 ignored rows."""
    import numpy as np
    rows = {0, n - 1}
    for c in range(chunk, n, chunk):
        rows.update({c - 1, c})
    rows.update(int(r) for r in rng.choice(n, size=min(16, n), replace=False))
    ign = np.flatnonzero(y == -100)
    if ign.size:
        rows.update(int(r) for r in rng.choice(ign, size=min(4, ign.size), replace=False))
    return sorted(r for r in rows if 0 <= r < n)


def sample_vocab(v, y, rng):
    """Vocabulary rows of dW the parity check compares: both ends, 6 label ids, 6 random ids."""
    cols = {0, 1, v - 1, v - 2}
    valid = y[y >= 0]
    if valid.size:
        cols.update(int(c) for c in rng.choice(valid, size=min(6, valid.size), replace=False))
    cols.update(int(c) for c in rng.choice(v, size=min(6, v), replace=False))
    return sorted(c for c in cols if 0 <= c < v)


def gpu_samples(torch, out, rows, cols):
    """Host copies of what the parity check compares: loss, every LSE, sampled dH and dW rows."""
    loss, lse, dh, dw = out
    dev = dh.device
    return {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
            "dh": dh[torch.as_tensor(rows, device=dev)].float().double().cpu().numpy(),
            "dw": dw[torch.as_tensor(cols, device=dev)].float().double().cpu().numpy(),
            "dh_ignored_zero": None}


def parity_against_oracle(wl, h, w, y, got, rows, cols, workers):
    """Errors of the GPU results against the fp64 oracle: the loss and every row's LSE from
    the oracle's whole forward, dH on sampled token rows and dW on sampled vocabulary rows
    (from the oracle's own LSE); the norms and tolerances of the parity tests."""
    import numpy as np

    from oracle import flce_dw_rows, flce_forward, flce_rows
    t0 = time.perf_counter()
    w64 = w.float().double().numpy() if hasattr(w, "numpy") else w
    rloss, rlse = flce_forward(h, w64, y, reduction=wl.reduction, workers=workers)
    _, rdh = flce_rows(h, w64, y, rows, reduction=wl.reduction)
    rdw = flce_dw_rows(h, w64, y, rlse, cols, reduction=wl.reduction)

    def rel_max(a, b):
        den = float(np.max(np.abs(b)))
        return float(np.max(np.abs(a - b))) / den if den > 0 else float(np.max(np.abs(a - b)))
    tol = {"bf16": (2e-3, 2e-2), "f32": (1e-5, 1e-4)}[wl.dtype]
    e = {"loss_rel": abs(got["loss"] - rloss) / abs(rloss) if rloss != 0 else abs(got["loss"] - rloss),
         "lse_max_rel": float(np.max(np.abs(got["lse"] - rlse) / np.abs(rlse))),
         "dh_rel_sampled": rel_max(got["dh"], rdh), "dw_rel_sampled": rel_max(got["dw"], rdw),
         "rows_sampled": len(rows), "vocab_rows_sampled": len(cols),
         "tolerance": {"loss_lse": tol[0], "grad": tol[1]}}
    e["within_tolerance"] = bool(e["loss_rel"] <= tol[0] and e["lse_max_rel"] <= tol[0]
                                 and e["dh_rel_sampled"] <= tol[1] and e["dw_rel_sampled"] <= tol[1])
    e["oracle_s"] = time.perf_counter() - t0
    return e


def measure_workload(flce, torch, wl, args, stream, h, w, y, with_kernels=False):
    """flce_fwd_bwd on one workload: uninstrumented per-step times, the pool's peak and
    reserved bytes, optionally a second instrumented pass (per-kernel times), and the
    host copies the parity check needs."""
    import numpy as np

    from workloads import logits_bytes_avoided
    dev = torch.device("cuda:0")
    hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
    o = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(wl.n, dtype=torch.float32, device=dev),
         torch.empty_like(hd), torch.empty_like(wd))
    dt = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    plan = flce.flce_plan_info(wl.n, wl.d, wl.v, dt, 1)

    def step():
        flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=o)
    step()
    torch.cuda.synchronize()
    flce.flce_memory_high_water(reset=True)
    per, total = time_steps(torch, step, stream, args.steps, max(1, args.warmup))
    extra = flce.flce_memory_high_water()
    reserved = flce.flce_memory_reserved()
    flop = 6.0 * wl.n * wl.d * wl.v
    res = {"n": wl.n, "d": wl.d, "v": wl.v, "dtype": wl.dtype, "reduction": wl.reduction,
           "ms_per_step": total / args.steps, "ms_median": median(per), "ms_min": min(per),
           "tokens_per_s": wl.n * args.steps / (total * 1e-3),
           "mfma_pct": 100.0 * flop / (total / args.steps * 1e-3) / (PEAK_TFLOPS[wl.dtype] * 1e12),
           "extra_device_bytes": extra, "pool_reserved_bytes": reserved,
           "logits_bytes_avoided": logits_bytes_avoided(wl.n, wl.v),
           "memory_ratio": extra / logits_bytes_avoided(wl.n, wl.v), "plan": plan}
    if with_kernels:
        flce.flce_profile_read()
        flce.flce_profile_enable(True)
        _, total_i = time_steps(torch, step, stream, args.steps, 0)
        flce.flce_profile_enable(False)
        res["ms_per_step_instrumented"] = total_i / args.steps
        res["kernels"] = flce.flce_profile_read()
    rng = np.random.default_rng(4242)
    rows = sample_rows(wl.n, plan["chunk_rows"], y.numpy(), rng)
    cols = sample_vocab(wl.v, y.numpy(), rng)
    got = gpu_samples(torch, o, rows, cols)
    ign = torch.from_numpy(y.numpy() == -100).to(dev)
    res["ignored_rows_dh_zero"] = bool((o[2][ign] == 0).all()) if bool(ign.any()) else None
    log(f"[bench] {wl.name}: {res['ms_per_step']:.3f} ms/step (median {res['ms_median']:.3f}), "
        f"{res['mfma_pct']:.1f}% of the {wl.dtype} peak, extra {extra / 1e6:.1f} MB "
        f"({res['memory_ratio']:.3f} of the fp32 logits)")
    handles = (hd, wd, yd, o)
    return res, got, rows, cols, handles


def lowmem_measure(flce, torch, wl, args, stream, hd, wd, yd, budgets):
    """flce_fwd_bwd_lowmem (forward statistics, then the backward over vocabulary slices
    with the logits recomputed): per budget of the slice buffer, the step time and the
    pool's peak against the fp32 logits; credited 6 N D V like the fused call."""
    from workloads import logits_bytes_avoided
    o = (torch.empty(1, dtype=torch.float32, device=hd.device), torch.empty(wl.n, dtype=torch.float32, device=hd.device),
         torch.empty_like(hd), torch.empty_like(wd))
    dt = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    out = []
    for b in budgets:
        if b is not None:
            os.environ["FLCE_LOWMEM_BUFFER_BYTES"] = str(b)
        try:
            plan = flce.flce_lowmem_plan_info(wl.n, wl.d, wl.v, dt)

            def step():
                flce.linear_cross_entropy_lowmem(hd, wd, yd, reduction=wl.reduction, out=o)
            step()
            torch.cuda.synchronize()
            flce.flce_memory_high_water(reset=True)
            _, total = time_steps(torch, step, stream, max(3, args.steps // 2), 1)
            peak = flce.flce_memory_high_water()
        finally:
            os.environ.pop("FLCE_LOWMEM_BUFFER_BYTES", None)
        ms = total / max(3, args.steps // 2)
        out.append({"path": "flce_fwd_bwd_lowmem", "slice_budget_bytes": plan["buffer_budget_bytes"],
                    "slices": plan["num_slices"], "slice_cols": plan["slice_cols"], "ms_per_step": ms,
                    "tokens_per_s": wl.n / (ms * 1e-3),
                    "mfma_pct_6ndv": 100.0 * 6.0 * wl.n * wl.d * wl.v / (ms * 1e-3) / (PEAK_TFLOPS[wl.dtype] * 1e12),
                    "mfma_pct_8ndv": 100.0 * 8.0 * wl.n * wl.d * wl.v / (ms * 1e-3) / (PEAK_TFLOPS[wl.dtype] * 1e12),
                    "extra_device_bytes": peak, "memory_ratio": peak / logits_bytes_avoided(wl.n, wl.v)})
        log(f"[bench] {wl.name} lowmem budget {plan['buffer_budget_bytes'] >> 20} MiB: {ms:.3f} ms/step, "
            f"peak {peak / 1e6:.1f} MB ({out[-1]['memory_ratio']:.3f})")
    return out


def fused_cap_measure(flce, torch, wl, args, stream, hd, wd, yd, caps):
    """flce_fwd_bwd under smaller chunk-buffer budgets (FLCE_WORKSPACE_CAP_BYTES): step
    time against the pool's peak."""
    from workloads import logits_bytes_avoided
    o = (torch.empty(1, dtype=torch.float32, device=hd.device), torch.empty(wl.n, dtype=torch.float32, device=hd.device),
         torch.empty_like(hd), torch.empty_like(wd))
    dt = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    out = []
    for cap in caps:
        os.environ["FLCE_WORKSPACE_CAP_BYTES"] = str(cap)
        try:
            plan = flce.flce_plan_info(wl.n, wl.d, wl.v, dt, 1)

            def step():
                flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=o)
            step()
            torch.cuda.synchronize()
            flce.flce_memory_high_water(reset=True)
            _, total = time_steps(torch, step, stream, max(3, args.steps // 2), 1)
            peak = flce.flce_memory_high_water()
        finally:
            os.environ.pop("FLCE_WORKSPACE_CAP_BYTES", None)
        ms = total / max(3, args.steps // 2)
        out.append({"path": "flce_fwd_bwd", "chunk_budget_bytes": cap, "chunk_rows": plan["chunk_rows"],
                    "chunks": plan["num_chunks"], "ms_per_step": ms, "tokens_per_s": wl.n / (ms * 1e-3),
                    "mfma_pct_6ndv": 100.0 * 6.0 * wl.n * wl.d * wl.v / (ms * 1e-3) / (PEAK_TFLOPS[wl.dtype] * 1e12),
                    "extra_device_bytes": peak, "memory_ratio": peak / logits_bytes_avoided(wl.n, wl.v)})
        log(f"[bench] {wl.name} fused, chunk budget {cap >> 20} MiB ({plan['chunk_rows']} rows): {ms:.3f} ms/step, "
            f"peak {peak / 1e6:.1f} MB ({out[-1]['memory_ratio']:.3f})")
    return out


def fp8_forward_measure(flce, torch, wl, args, stream):
    """flce_fwd_fp8 on this workload's H and W quantised row by row to e4m3:
    2 N D V flop against the fp8 matrix peak."""
    from workloads import make_inputs_fp8
    hq, hs, wq, ws, y = make_inputs_fp8(wl)
    dev = torch.device("cuda:0")
    hq, hs, wq, ws, y = hq.to(dev), hs.to(dev), wq.to(dev), ws.to(dev), y.to(dev)
    for _ in range(max(1, args.warmup)):
        flce.linear_cross_entropy_forward_fp8(hq, hs, wq, ws, y, reduction=wl.reduction)
    torch.cuda.synchronize()
    flce.flce_profile_read()
    flce.flce_profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        flce.linear_cross_entropy_forward_fp8(hq, hs, wq, ws, y, reduction=wl.reduction)
    e1.record(stream)
    torch.cuda.synchronize()
    flce.flce_profile_enable(False)
    kern = flce.flce_profile_read()
    ms = e0.elapsed_time(e1) / args.steps
    flop = 2.0 * wl.n * wl.d * wl.v
    launches, lg_ms = kern.get("logits_lse", (0, 0.0))
    lg_avg = lg_ms / max(launches, 1)
    flop_launch = flop / max(launches // args.steps, 1)
    log(f"[bench] fp8 forward: {ms:.3f} ms/call, logits launch {lg_avg:.3f} ms")
    out = {
        "ms_per_call": ms,
        "tflops_2ndv": flop / (ms * 1e-3) / 1e12,
        "peak_tflops": PEAK_TFLOPS["fp8"],
        "mfma_pct_2ndv": 100.0 * flop / (ms * 1e-3) / (PEAK_TFLOPS["fp8"] * 1e12),
        "logits_launch_ms": lg_avg,
        "logits_frac": flop_launch / (lg_avg * 1e-3) / (PEAK_TFLOPS["fp8"] * 1e12),
        "inputs": "H and W quantised per row to e4m3 (scale max|row|/448)",
    }
    out["backward"] = fp8_backward_measure(flce, torch, wl, args, stream, (hq, hs, wq, ws, y))
    return out


def fp8_backward_measure(flce, torch, wl, args, stream, inputs):
    """flce_bwd_fp8 from the forward's LSE: the fp8 logits recompute (2 N D V flop at the
    fp8 peak) plus dH and dW on the dequantised bf16 copies (4 N D V at the bf16 peak).
    `ideal_ms` is the time of that work at the two peaks; `frac` = ideal / measured."""
    hq, hs, wq, ws, y = inputs
    _, lse = flce.linear_cross_entropy_forward_fp8(hq, hs, wq, ws, y, reduction=wl.reduction)
    go = torch.ones(1, dtype=torch.float32, device=hq.device)
    for _ in range(max(1, args.warmup)):
        flce.linear_cross_entropy_backward_fp8(hq, hs, wq, ws, y, lse, go, reduction=wl.reduction)
    torch.cuda.synchronize()
    flce.flce_profile_read()
    flce.flce_profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        flce.linear_cross_entropy_backward_fp8(hq, hs, wq, ws, y, lse, go, reduction=wl.reduction)
    e1.record(stream)
    torch.cuda.synchronize()
    flce.flce_profile_enable(False)
    kern = flce.flce_profile_read()
    ms = e0.elapsed_time(e1) / args.steps
    ndv = float(wl.n) * wl.d * wl.v
    ideal = (2.0 * ndv / (PEAK_TFLOPS["fp8"] * 1e12) + 4.0 * ndv / (PEAK_TFLOPS["bf16"] * 1e12)) * 1e3
    per_call = {k: ms_k / args.steps for k, (cnt, ms_k) in kern.items() if cnt}
    log(f"[bench] fp8 backward: {ms:.3f} ms/call ({100.0 * ideal / ms:.1f}% of the mixed peak), kernels {per_call}")
    return {"ms_per_call": ms, "ideal_ms": ideal, "frac": ideal / ms, "kernel_ms_per_call": per_call,
            "flop": "2NDV fp8 (logits recompute) + 4NDV bf16 (dH, dW)"}


def vendor_gemm_measure(torch, hd, wd, yd, wl, args, stream, chunk):
    """torch's own bf16 matrix products (hipBLASLt) on the three contraction shapes of
    one chunk of `chunk` tokens: Z = H_c W^T, dH_c = G W and dW = G^T H_c, with G the
    real softmax-minus-one-hot gradient of that chunk.  Context for the library's
    contraction kernels on the same chip and clock limits, not a path of the library."""
    c = min(chunk, wl.n)
    hc = hd[:c].contiguous()
    z = torch.matmul(hc, wd.t())
    g = torch.softmax(z.float(), dim=-1)
    yc = yd[:c]
    keep = yc != -100
    rows = torch.arange(c, device=hd.device)[keep]
    g[rows, yc[keep]] -= 1.0
    g = (g / max(1, int((yd != -100).sum()))).to(z.dtype)
    gt = g.t().contiguous()                    # dW's left operand, laid out as the library reads it
    flop = 2.0 * c * wl.d * wl.v
    peak = PEAK_TFLOPS[wl.dtype]
    res = {"chunk_rows": c, "flop_per_product": flop, "library": "torch.matmul (hipBLASLt)",
           "g": "softmax(H_c W^T) minus one-hot, divided by the valid-token count, bf16"}
    prods = {"logits_z": lambda: torch.matmul(hc, wd.t()),
             "dh_gw": lambda: torch.matmul(g, wd),
             "dw_gth": lambda: torch.matmul(gt, hc)}
    total = 0.0
    for name, fn in prods.items():
        _, tot = time_steps(torch, fn, stream, args.steps, max(1, args.warmup))
        ms = tot / args.steps
        total += ms
        res[name] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12, "frac": flop / (ms * 1e-3) / (peak * 1e12)}
        log(f"[bench] hipBLASLt {name}: {ms:.3f} ms ({res[name]['tflops']:.0f} TFLOP/s, "
            f"{100 * res[name]['frac']:.1f}% of peak)")
    res["three_products_ms"] = total
    res["frac_three_products"] = 3 * flop / (total * 1e-3) / (peak * 1e12)
    del z, g, gt, hc
    return res


def ce_logits_measure(flce, torch, hd, wd, yd, wl, args, stream):
    """Cross-entropy on materialised logits (flce_ce_logits) for this workload's
    logits Z = H W^T: forward only, forward + gradient into a separate buffer,
    and the backward from the saved LSE.  HBM-bound; the algorithmic bytes are
    one read of Z (forward) and one read of Z plus one write of the gradient
    (gradient modes)."""
    n, v = wl.n, wl.v
    z = torch.matmul(hd, wd.t())             # input preparation only, outside the timed region
    g = torch.empty_like(z)
    loss = torch.empty(1, dtype=torch.float32, device=hd.device)
    lse = torch.empty(n, dtype=torch.float32, device=hd.device)
    dt_code = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    red_code = flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM
    elem = z.element_size()
    modes = {
        "forward": (lambda: flce.flce_ce_logits(z, yd, n, v, dt_code, -100, red_code, None, None, loss, lse, None,
                                                stream), n * v * elem),
        "forward_grad": (lambda: flce.flce_ce_logits(z, yd, n, v, dt_code, -100, red_code, None, None, loss, lse, g,
                                                     stream), 2 * n * v * elem),
        "backward_from_lse": (lambda: flce.flce_ce_logits(z, yd, n, v, dt_code, -100, red_code, lse, None, None,
                                                          None, g, stream), 2 * n * v * elem),
    }
    res = {"workload": f"{wl.name} logits [{n}, {v}] {wl.dtype}", "peak_GBps": HBM_PEAK_GBPS}
    for name, (fn, nbytes) in modes.items():
        for _ in range(max(1, args.warmup)):
            if fn() != flce.FLCE_OK:
                raise RuntimeError(f"flce_ce_logits {name} failed")
        torch.cuda.synchronize()
        flce.flce_profile_read()
        flce.flce_profile_enable(True)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        flce.flce_profile_enable(False)
        kern = flce.flce_profile_read()
        launches, ms = kern.get("ce_rows", (0, 0.0))
        avg = ms / max(launches, 1)
        res[name] = {"ce_rows_avg_ms": avg, "algorithmic_bytes": nbytes,
                     "traffic": measured_traffic("ce_fwd_grad") if name == "forward_grad" else None,
                     "achieved_GBps": nbytes / (avg * 1e-3) / 1e9,
                     "frac": nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "ms_per_call": sum(t for _, t in kern.values()) / args.steps}
        log(f"[bench] ce_logits {name}: {avg:.3f} ms ({res[name]['achieved_GBps']:.0f} GB/s)")
    # practical ceiling: a device-to-device copy of the same bytes (one read + one write)
    for _ in range(2):
        g.copy_(z)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(args.steps):
        g.copy_(z)
    c1.record(stream)
    torch.cuda.synchronize()
    ms_copy = c0.elapsed_time(c1) / args.steps
    res["device_copy"] = {"ms": ms_copy, "GBps": 2 * n * v * elem / (ms_copy * 1e-3) / 1e9}
    log(f"[bench] device copy of the logits: {ms_copy:.3f} ms ({res['device_copy']['GBps']:.0f} GB/s)")
    del z, g
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama3_8b_head")
    ap.add_argument("--cpu-rows", type=int, default=6144, help="tokens in the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other four workloads (by default every workload is timed and reported)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the comparison with the fp64 oracle (by default every workload is checked)")
    ap.add_argument("--no-memory-sweep", action="store_true",
                    help="skip the low-memory path and the chunk-budget sweep")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload's flce_fwd_bwd (no other entry points, workloads "
                         "or sweeps), so that a profiler's per-kernel averages cover the headline launches "
                         "alone")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB device copy (counter calibration), one step and one cross-entropy on "
                         "the workload's logits, print nothing else; meant to run under rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.headline_only:
        args.no_per_config = args.no_memory_sweep = True

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fused linear cross-entropy path here has no multi-GPU "
              "mode (it would shard by tokens, with one all-reduce of dW, or by vocabulary rows, with an "
              "all-gather of the per-token LSE partials); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import linear_cross_entropy_bwd_amd as flce
    from workloads import CONFIGS, logits_bytes_avoided, make_inputs

    wl = CONFIGS[args.config]
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    log(f"[bench] generating {wl.name}: n={wl.n} d={wl.d} v={wl.v} {wl.dtype}")
    h, w, y = make_inputs(wl)
    plan = flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32, 1)
    log(f"[bench] plan {plan}")

    if args.traffic_probe:
        hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
        out = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(wl.n, dtype=torch.float32, device=dev),
               torch.empty_like(hd), torch.empty_like(wd))
        for i in range(args.warmup):
            flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
        torch.cuda.synchronize()
        log(f"[bench] {args.warmup} warm-up steps done")
        # A plain copy of exactly COPY_BYTES (read COPY_BYTES, write COPY_BYTES) calibrates
        # the FETCH_SIZE / WRITE_SIZE counters against a known byte count.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
        torch.cuda.synchronize()
        # and one cross-entropy on this workload's logits, forward + gradient into a separate buffer
        z = torch.matmul(hd, wd.t())
        g = torch.empty_like(z)
        loss_z = torch.empty(1, dtype=torch.float32, device=dev)
        lse_z = torch.empty(wl.n, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        st = flce.flce_ce_logits(z, yd, wl.n, wl.v, flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32, -100,
                                 flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM, None, None, loss_z,
                                 lse_z, g, torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        if st != flce.FLCE_OK:
            raise flce.FlceError(st, "flce_ce_logits")
        log("[bench] traffic probe done")
        return 0

    stream = torch.cuda.current_stream(dev)
    # The headline: flce_fwd_bwd on this workload, timed without instrumentation, then a
    # second, instrumented pass for the per-kernel split (the roofline's dominant kernel).
    head, head_got, head_rows, head_cols, handles = measure_workload(flce, torch, wl, args, stream, h, w, y,
                                                                     with_kernels=True)
    kern = head["kernels"]
    ms_step = head["ms_per_step"]
    flops_step = 6.0 * wl.n * wl.d * wl.v
    peak = PEAK_TFLOPS[wl.dtype]
    # dominant kernel: the contraction kind with the largest total time
    dom = max(GEMM_KINDS, key=lambda k: kern.get(k, (0, 0.0))[1])
    launches, dom_ms = kern[dom]
    flops_launch = 2.0 * wl.n * wl.d * wl.v / plan["num_chunks"]      # 2*C*D*V per chunk launch (avg)
    dom_avg_ms = dom_ms / max(launches, 1)
    achieved = flops_launch / (dom_avg_ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step uninstrumented (median {head['ms_median']:.3f}, "
        f"min {head['ms_min']:.3f}), {head['ms_per_step_instrumented']:.3f} instrumented; kernels {kern}")

    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": head["ms_median"],
        "ms_per_step_min": head["ms_min"],
        "ms_per_step_instrumented": head["ms_per_step_instrumented"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded: H~N(0,1), W~N(0,0.02^2), uniform labels, 5% ignore_index)",
        "config": {"workload": wl.name, "n": wl.n, "d": wl.d, "v": wl.v, "reduction": wl.reduction,
                   "ignored_frac": wl.ignore_frac, "parallelism": "none (1 GPU)"},
        "mfma_pct": 100.0 * flops_step / (ms_step * 1e-3) / (peak * 1e12),
        "tflops": flops_step / (ms_step * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic(dom),
                     "avg_launch_ms": dom_avg_ms, "flop_per_launch": flops_launch,
                     "timing": "HIP events around each launch on the call's stream (instrumented pass)"},
        "kernels_ms_per_step": {k: v[1] / args.steps for k, v in kern.items() if v[0]},
        "kernels_ms_per_launch": {k: v[1] / v[0] for k, v in kern.items() if v[0]},
        "memory": {"extra_device_bytes": head["extra_device_bytes"],
                   "pool_reserved_bytes": head["pool_reserved_bytes"],
                   "logits_bytes_avoided": logits_bytes_avoided(wl.n, wl.v),
                   "ratio": head["memory_ratio"]},
        "plan": plan,
    }
    hd, wd, yd, out = handles
    dt_code = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    red_code = flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM
    loss_s, lse_s, dh_s, dw_s = out

    # The low-memory path and the memory/speed trade-off on this workload.
    if not args.no_memory_sweep:
        lm = lowmem_measure(flce, torch, wl, args, stream, hd, wd, yd, [None, 128 << 20, 512 << 20])
        result["lowmem"] = lm[0]
        result["memory_tradeoff"] = {"workload": wl.name, "points": fused_cap_measure(
            flce, torch, wl, args, stream, hd, wd, yd, [1 << 30, 512 << 20, 256 << 20]) + lm}

    # The other entry points on this workload (skipped with --headline-only).
    if not args.headline_only:
        # The split path an autograd function uses: flce_fwd (loss, LSE) then flce_bwd
        # (logits recomputed from the saved LSE), 8 N D V flop per step.
        def split_step():
            st = flce.flce_fwd(hd, wd, yd, wl.n, wl.d, wl.v, dt_code, -100, red_code, loss_s, lse_s, stream)
            st = st or flce.flce_bwd(hd, wd, yd, lse_s, None, wl.n, wl.d, wl.v, dt_code, -100, red_code, dh_s, dw_s,
                                     stream)
            if st != flce.FLCE_OK:
                raise flce.FlceError(st, "split step")

        _, tot = time_steps(torch, split_step, stream, args.steps, max(1, args.warmup))
        ms_split = tot / args.steps
        log(f"[bench] split fwd + bwd-from-LSE: {ms_split:.3f} ms/step")
        result["split_fwd_bwd"] = {
            "ms_per_step": ms_split,
            "tokens_per_s": wl.n / (ms_split * 1e-3),
            "tflops_8ndv": 8.0 * wl.n * wl.d * wl.v / (ms_split * 1e-3) / 1e12,
            "mfma_pct_8ndv": 100.0 * 8.0 * wl.n * wl.d * wl.v / (ms_split * 1e-3) / (peak * 1e12),
            "path": "flce_fwd then flce_bwd (logits recomputed from the saved LSE)",
        }

        # flce_fwd_bwd with the softmax factor written into the stored probabilities in
        # place (FLCE_INPLACE_GRAD=1) instead of applied per row, for comparison
        os.environ["FLCE_INPLACE_GRAD"] = "1"
        try:
            def inplace_step():
                flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
            inplace_step()
            torch.cuda.synchronize()
            flce.flce_memory_high_water(reset=True)
            _, tot = time_steps(torch, inplace_step, stream, args.steps, max(1, args.warmup))
            peak_ip = flce.flce_memory_high_water()
        finally:
            os.environ.pop("FLCE_INPLACE_GRAD", None)
        ms_ip = tot / args.steps
        log(f"[bench] fused, in-place gradient pass: {ms_ip:.3f} ms/step, peak {peak_ip / 1e6:.1f} MB")
        result["inplace_grad"] = {
            "ms_per_step": ms_ip,
            "tokens_per_s": wl.n / (ms_ip * 1e-3),
            "mfma_pct_6ndv": 100.0 * 6.0 * wl.n * wl.d * wl.v / (ms_ip * 1e-3) / (peak * 1e12),
            "extra_device_bytes": peak_ip,
            "path": "flce_fwd_bwd, FLCE_INPLACE_GRAD=1 (P rewritten into G in place; no per-row factor)",
        }

        # the forward alone (loss and LSE), 2 N D V flop
        def fwd_only():
            st = flce.flce_fwd(hd, wd, yd, wl.n, wl.d, wl.v, dt_code, -100, red_code, loss_s, lse_s, stream)
            if st != flce.FLCE_OK:
                raise flce.FlceError(st, "flce_fwd")

        _, tot = time_steps(torch, fwd_only, stream, args.steps, max(1, args.warmup))
        ms_fwd = tot / args.steps
        log(f"[bench] forward only: {ms_fwd:.3f} ms/call")
        result["forward_only"] = {
            "ms_per_call": ms_fwd,
            "tokens_per_s": wl.n / (ms_fwd * 1e-3),
            "tflops_2ndv": 2.0 * wl.n * wl.d * wl.v / (ms_fwd * 1e-3) / 1e12,
            "mfma_pct_2ndv": 100.0 * 2.0 * wl.n * wl.d * wl.v / (ms_fwd * 1e-3) / (peak * 1e12),
            "path": "flce_fwd (loss and LSE; logits statistics only)",
        }

        # vocabulary split in eight shards (the shard shape of an eight-way vocabulary-parallel
        # head): per shard the partial forward, the merge, per shard the backward from the merged
        # LSE, the sum of the dH terms; 8 N D V flop
        def split8():
            flce.linear_cross_entropy_vocab_split(hd, wd, yd, num_shards=8, reduction=wl.reduction)

        _, tot = time_steps(torch, split8, stream, args.steps, max(1, args.warmup))
        ms_vs = tot / args.steps
        log(f"[bench] vocabulary split, 8 shards: {ms_vs:.3f} ms/step")
        result["vocab_split_8"] = {
            "ms_per_step": ms_vs,
            "tokens_per_s": wl.n / (ms_vs * 1e-3),
            "tflops_8ndv": 8.0 * wl.n * wl.d * wl.v / (ms_vs * 1e-3) / 1e12,
            "mfma_pct_8ndv": 100.0 * 8.0 * wl.n * wl.d * wl.v / (ms_vs * 1e-3) / (peak * 1e12),
            "shards": flce.vocab_shard_bounds(wl.v, 8),
            "path": "flce_fwd_shard x8, flce_merge_shards, flce_bwd_shard x8, flce_sum_parts",
        }
        result["forward_fp8"] = fp8_forward_measure(flce, torch, wl, args, stream)
        result["ce_logits"] = ce_logits_measure(flce, torch, hd, wd, yd, wl, args, stream)
        result["vendor_gemm"] = vendor_gemm_measure(torch, hd, wd, yd, wl, args, stream, plan["chunk_rows"])
    del hd, wd, yd, out, loss_s, lse_s, dh_s, dw_s, handles
    torch.cuda.empty_cache()

    # Every workload: flce_fwd_bwd timed the same way; results kept on the host for parity.
    pending = [(wl, h, w, y, head_got, head_rows, head_cols)]
    per_config = {wl.name: {k: v for k, v in head.items() if k not in ("kernels",)}}
    if not args.no_per_config:
        for name, other in CONFIGS.items():
            if name == wl.name:
                continue
            log(f"[bench] generating {name}: n={other.n} d={other.d} v={other.v} {other.dtype}")
            ho, wo, yo = make_inputs(other)
            res, got, rows, cols, hh = measure_workload(flce, torch, other, args, stream, ho, wo, yo)
            del hh
            torch.cuda.empty_cache()
            per_config[name] = res
            pending.append((other, ho, wo, yo, got, rows, cols))
    result["per_config"] = per_config

    # Parity against the fp64 oracle (host cores), after all GPU timing.
    if not args.no_parity:
        workers = min(16, len(os.sched_getaffinity(0)))
        for owl, ho, wo, yo, got, rows, cols in pending:
            par = parity_against_oracle(owl, ho, wo, yo, got, rows, cols, workers)
            per_config[owl.name]["parity"] = par
            log(f"[bench] parity {owl.name}: loss {par['loss_rel']:.2e}, lse {par['lse_max_rel']:.2e}, "
                f"dH {par['dh_rel_sampled']:.2e}, dW {par['dw_rel_sampled']:.2e} ({par['oracle_s']:.1f} s)")
        result["parity"] = per_config[wl.name]["parity"]
    del pending

    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle on {args.cpu_rows} rows")
        result["cpu_baseline"] = cpu_baseline(wl, h, w, y, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
