"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

One step = one flce_fwd_bwd call (label scan, logits GEMM with the online
LSE / target epilogue, merge, in-place gradient, dH and dW GEMMs, loss
reduction) over the Llama-3-8B LM-head workload: N=8192 tokens, D=4096,
V=128256, bf16, 5% ignored labels, mean reduction.  Inputs are synthetic,
seeded and resident in HBM before timing starts.

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


def all_configs_measure(flce, torch, args, stream):
    """flce_fwd_bwd on every workload: median step time, tokens/s, MFMA % (6 N D V against
    the workload dtype's matrix peak) and the extra device memory against the N V 4 bytes
    of logits it avoids."""
    from workloads import CONFIGS, logits_bytes_avoided, make_inputs
    out = {}
    for name, wl in CONFIGS.items():
        h, w, y = make_inputs(wl)
        dev = torch.device("cuda:0")
        hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
        del h, w
        o = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(wl.n, dtype=torch.float32, device=dev),
             torch.empty_like(hd), torch.empty_like(wd))
        for _ in range(max(1, args.warmup)):
            flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=o)
        torch.cuda.synchronize()
        flce.flce_memory_high_water(reset=True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for i in range(args.steps):
            flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=o)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        extra = flce.flce_memory_high_water()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
        flop = 6.0 * wl.n * wl.d * wl.v
        out[name] = {"n": wl.n, "d": wl.d, "v": wl.v, "dtype": wl.dtype, "ms_median": med, "ms_min": t[0],
                     "tokens_per_s": wl.n / (med * 1e-3),
                     "mfma_pct": 100.0 * flop / (med * 1e-3) / (PEAK_TFLOPS[wl.dtype] * 1e12),
                     "extra_device_bytes": extra, "logits_bytes_avoided": logits_bytes_avoided(wl.n, wl.v)}
        log(f"[bench] {name}: {med:.3f} ms median, {out[name]['mfma_pct']:.1f}% of the {wl.dtype} peak")
        del hd, wd, yd, o
        torch.cuda.empty_cache()
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
    ap.add_argument("--all-configs", action="store_true",
                    help="also time flce_fwd_bwd on every workload (inputs drawn per workload) and report each")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB device copy (counter calibration), one step and one cross-entropy on "
                         "the workload's logits, print nothing else; meant to run under rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

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
    hd, wd, yd = h.to(dev), w.to(dev), y.to(dev)
    out = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(wl.n, dtype=torch.float32, device=dev),
           torch.empty_like(hd), torch.empty_like(wd))
    plan = flce.flce_plan_info(wl.n, wl.d, wl.v, flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32, 1)
    log(f"[bench] plan {plan}")

    for i in range(args.warmup):
        flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warm-up steps done")

    if args.traffic_probe:
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

    # peak extra device memory of one call
    flce.flce_memory_high_water(reset=True)
    flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
    torch.cuda.synchronize()
    extra = flce.flce_memory_high_water()

    stream = torch.cuda.current_stream(dev)
    flce.flce_profile_read()                 # clear
    flce.flce_profile_enable(True)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        flce.linear_cross_entropy(hd, wd, yd, reduction=wl.reduction, out=out)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    flce.flce_profile_enable(False)
    kern = flce.flce_profile_read()
    ms_total = ev[0].elapsed_time(ev[-1])
    ms_step = ms_total / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (
        per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (median {ms_median:.3f}, min {per_step[0]:.3f}; "
        f"wall {wall:.2f} s); kernels {kern}")

    flops_step = 6.0 * wl.n * wl.d * wl.v
    peak = PEAK_TFLOPS[wl.dtype]
    # dominant kernel: the contraction kind with the largest total time
    dom = max(GEMM_KINDS, key=lambda k: kern.get(k, (0, 0.0))[1])
    launches, dom_ms = kern[dom]
    flops_launch = 2.0 * wl.n * wl.d * wl.v / plan["num_chunks"]      # 2*C*D*V per chunk launch (avg)
    dom_avg_ms = dom_ms / max(launches, 1)
    achieved = flops_launch / (dom_avg_ms * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": wl.n * args.steps / (ms_total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_median,
        "ms_per_step_min": per_step[0],
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
                     "avg_launch_ms": dom_avg_ms, "flop_per_launch": flops_launch},
        "kernels_ms_per_step": {k: v[1] / args.steps for k, v in kern.items() if v[0]},
        "memory": {"extra_device_bytes": extra, "logits_bytes_avoided": logits_bytes_avoided(wl.n, wl.v),
                   "ratio": extra / logits_bytes_avoided(wl.n, wl.v)},
        "plan": plan,
    }
    # The split path an autograd function uses: flce_fwd (loss, LSE) then flce_bwd
    # (logits recomputed from the saved LSE), 8 N D V flop per step.
    dt_code = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    red_code = flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM
    loss_s, lse_s, dh_s, dw_s = out

    def split_step():
        st = flce.flce_fwd(hd, wd, yd, wl.n, wl.d, wl.v, dt_code, -100, red_code, loss_s, lse_s, stream)
        st = st or flce.flce_bwd(hd, wd, yd, lse_s, None, wl.n, wl.d, wl.v, dt_code, -100, red_code, dh_s, dw_s,
                                 stream)
        if st != flce.FLCE_OK:
            raise flce.FlceError(st, "split step")

    for _ in range(max(1, args.warmup)):
        split_step()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(args.steps):
        split_step()
    s1.record(stream)
    torch.cuda.synchronize()
    ms_split = s0.elapsed_time(s1) / args.steps
    log(f"[bench] split fwd + bwd-from-LSE: {ms_split:.3f} ms/step")
    result["split_fwd_bwd"] = {
        "ms_per_step": ms_split,
        "tokens_per_s": wl.n / (ms_split * 1e-3),
        "tflops_8ndv": 8.0 * wl.n * wl.d * wl.v / (ms_split * 1e-3) / 1e12,
        "mfma_pct_8ndv": 100.0 * 8.0 * wl.n * wl.d * wl.v / (ms_split * 1e-3) / (peak * 1e12),
        "path": "flce_fwd then flce_bwd (logits recomputed from the saved LSE)",
    }
    # the forward alone (loss and LSE), 2 N D V flop
    def fwd_only():
        st = flce.flce_fwd(hd, wd, yd, wl.n, wl.d, wl.v, dt_code, -100, red_code, loss_s, lse_s, stream)
        if st != flce.FLCE_OK:
            raise flce.FlceError(st, "flce_fwd")

    for _ in range(max(1, args.warmup)):
        fwd_only()
    torch.cuda.synchronize()
    s0.record(stream)
    for _ in range(args.steps):
        fwd_only()
    s1.record(stream)
    torch.cuda.synchronize()
    ms_fwd = s0.elapsed_time(s1) / args.steps
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

    for _ in range(max(1, args.warmup)):
        split8()
    torch.cuda.synchronize()
    s0.record(stream)
    for _ in range(args.steps):
        split8()
    s1.record(stream)
    torch.cuda.synchronize()
    ms_vs = s0.elapsed_time(s1) / args.steps
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
    if args.all_configs:
        result["per_config"] = all_configs_measure(flce, torch, args, stream)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle on {args.cpu_rows} rows")
        result["cpu_baseline"] = cpu_baseline(wl, h, w, y, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
