"""Attention forward (and, with --backward, backward) throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mid]
    python bench.py --backward [--workload mid] [--causal]

One step is one fa_fwd call (the whole forward: Q load, K/V stream, QK^T,
masking, online softmax, PV, epilogue) over the workload's synthetic inputs,
already resident in HBM.  W untimed steps, then exactly K timed steps between
two device synchronisations; HIP events recorded on the launch stream give
the kernel's average duration.  FLOPs per step = 4*B*H*Lq*Lk*D (halved when
causal).  Prints one JSON line.

Extra fields: ``roofline`` (MFMA-bound; achieved TFLOP/s of the kernel vs the
published 2.5 PFLOP/s dense bf16 peak, and HBM traffic from the committed
rocprofv3 counter summary when it matches the current kernel source),
``cpu_baseline`` (the fp64 CPU oracle timed on a bounded row sample of the
same workload), ``parity`` (sampled rows of this run's output against the
oracle) and, with --secondary, ``secondary`` (the 16K non-causal forward,
the other shape the metric names).

With --backward one step is one fa_bwd call (the delta, dK/dV and dQ kernels
in order on one stream) over the same inputs plus a seeded dO, with o and lse
from one forward call made before timing.  FLOPs per step are the
algorithmic count of the five products (S, dP, dV, dK, dQ):
10*B*H*Lq*Lk*D, halved when causal, i.e. 2.5x the forward's; the kernels
recompute S and dP in both gradient kernels (7 products executed).  The
roofline entry times the whole call with HIP events on its stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak, D=128 N=4096/16384"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
KERNEL_SRC = os.path.join(ROOT, "scaled_dot_product_fa_amd", "csrc",
                          "fa_mfma.hip")
BWD_KERNEL_SRC = os.path.join(ROOT, "scaled_dot_product_fa_amd", "csrc",
                              "fa_bwd_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(src: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def workload_desc(w, causal):
    return (f"{w.name} B={w.B} H={w.H} Lq={w.Lq} Lk={w.Lk} D={w.D} {w.dtype} "
            f"{'causal' if causal else 'non-causal'}")


def visible_pairs(Lq, Lk, causal, window):
    """Number of (query, key) pairs the mask keeps."""
    import numpy as np
    i = np.arange(Lq, dtype=np.int64)
    lo = np.zeros(Lq, dtype=np.int64)
    hi = np.full(Lq, Lk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if window is not None and window[0] >= 0:
        lo = np.maximum(lo, i - window[0])
    if window is not None and window[1] >= 0:
        hi = np.minimum(hi, i + window[1])
    return int(np.maximum(hi - lo + 1, 0).sum())


def time_forward(w, causal, steps, warmup, layout="bhld", window=None):
    """Returns dict with wall ms/step, event ms/launch, flops and buffers.
    layout "blhd": the inputs live in [B, L, H, D] buffers (viewed as
    [B, H, L, D]); window (left, right): local mask.  Both go through
    fa_fwd_ex; FLOPs are then 4*D per kept (query, key) pair."""
    import torch
    import scaled_dot_product_fa_amd as fa
    from scaled_dot_product_fa_amd import inputs

    dev = torch.device("cuda:0")
    q, k, v = inputs.workload_inputs(w)
    if layout == "blhd":
        dq, dk, dv = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
                      for t in (q, k, v))
    else:
        dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Lq), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    name = fa.fa_kernel_name(w.B, w.H, w.Lq, w.Lk, w.D, int(causal), w.scale,
                             fa.dtype_code(dq.dtype))
    general = layout != "bhld" or window is not None
    if general:
        name = f"{name} via fa_fwd_ex ({layout}, window {window})"
        flops = 4.0 * w.B * w.H * w.D * visible_pairs(w.Lq, w.Lk, causal, window)
    else:
        flops = w.flops(causal)
    log(f"bench: {workload_desc(w, causal)} kernel={name} warmup={warmup} "
        f"steps={steps}")
    for _ in range(warmup):
        fa.forward(dq, dk, dv, causal=causal, scale=w.scale, out=o, lse=lse,
                   stream=stream, window=window)
    torch.cuda.synchronize(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fa.forward(dq, dk, dv, causal=causal, scale=w.scale, out=o, lse=lse,
                   stream=stream, window=window)
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    return dict(wall_ms=(t1 - t0) * 1e3 / steps,
                kernel_ms=ev0.elapsed_time(ev1) / steps,
                flops=flops, bytes=w.io_bytes(), kernel=name,
                q=q, k=k, v=v, o=o.contiguous(), lse=lse, window=window)


def time_backward(w, causal, steps, warmup, layout="bhld", window=None):
    """Backward: dict with wall ms/step, event ms/call, flops and buffers.
    layout / window as for time_forward (then fa_bwd_ex; FLOPs 10*D per
    kept pair)."""
    import torch
    import scaled_dot_product_fa_amd as fa
    from scaled_dot_product_fa_amd import inputs

    dev = torch.device("cuda:0")
    q, k, v = inputs.workload_inputs(w)
    g = inputs.make_dout(w.B, w.H, w.Lq, w.D, w.dtype, w.seed)
    if layout == "blhd":
        dq_, dk_, dv_, dg = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
                             for t in (q, k, v, g))
    else:
        dq_, dk_, dv_, dg = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
    stream = torch.cuda.current_stream(dev)
    o, lse = fa.forward(dq_, dk_, dv_, causal=causal, scale=w.scale, stream=stream,
                        window=window)
    gq, gk, gv = (torch.empty_like(t) for t in (dq_, dk_, dv_))
    delta = torch.empty_like(lse)
    name = fa.fa_bwd_kernel_name(w.B, w.H, w.Lq, w.Lk, w.D, int(causal), w.scale,
                                 fa.dtype_code(dq_.dtype))
    log(f"bench: backward {workload_desc(w, causal)} kernel={name} "
        f"warmup={warmup} steps={steps}")

    general = layout != "bhld" or window is not None
    if general:
        name = f"{name} via fa_bwd_ex ({layout}, window {window})"
        flops = 10.0 * w.B * w.H * w.D * visible_pairs(w.Lq, w.Lk, causal, window)
    else:
        flops = 2.5 * w.flops(causal)

    def step():
        fa.backward(dq_, dk_, dv_, o, lse, dg, causal=causal, scale=w.scale,
                    dq=gq, dk=gk, dv=gv, delta=delta, stream=stream, window=window)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    return dict(wall_ms=(t1 - t0) * 1e3 / steps,
                kernel_ms=ev0.elapsed_time(ev1) / steps,
                flops=flops, kernel=name, window=window,
                q=q, k=k, v=v, g=g, dq=gq, dk=gk, dv=gv)


def bwd_heads(w, n):
    """n heads (b, h) spread over the workload, seeded order."""
    step = max(1, (w.B * w.H) // n)
    return [(bh // w.H, bh % w.H) for bh in range(0, w.B * w.H, step)][:n]


def parity_bwd(w, causal, r):
    """Gradients of one sampled head against the oracle (error / max|ref|)."""
    import numpy as np
    import torch
    import oracle
    f64 = lambda t: t.to(torch.float64).numpy()
    (b, h), = bwd_heads(w, 1)[-1:]
    sl = (slice(b, b + 1), slice(h, h + 1))
    win = r.get("window")
    win = None if win is None else tuple(win)
    ref = oracle.attention_bwd(f64(r["q"][sl]), f64(r["k"][sl]), f64(r["v"][sl]),
                               f64(r["g"][sl]), causal, w.scale, window=win)
    out = {"head": [b, h]}
    for name, got, rr in zip(("dq", "dk", "dv"), (r["dq"], r["dk"], r["dv"]), ref):
        out[f"err_{name}"] = float(np.abs(f64(got[sl].cpu()) - rr).max()
                                   / max(np.abs(rr).max(), 1e-30))
    return out


def cpu_baseline_bwd(w, causal, r, budget_s=15.0):
    """The fp64 oracle backward on whole heads of the same workload (heads are
    independent), as many as fit the budget (at least one), scaled to
    TFLOP/s with the same algorithmic FLOP formula per head."""
    import torch
    import oracle
    f64 = lambda t: t.to(torch.float64).numpy()
    win = r.get("window")
    win = None if win is None else tuple(win)
    per_head = r["flops"] / (w.B * w.H)
    done, t_total = 0, 0.0
    for b, h in bwd_heads(w, w.B * w.H):
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [f64(r[x][sl]) for x in ("q", "k", "v", "g")]
        t0 = time.perf_counter()
        oracle.attention_bwd(*args, causal, w.scale, window=win)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    return dict(value=done * per_head / t_total / 1e12, unit="TFLOP/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=(f"{done} whole head(s) of {workload_desc(w, causal)} "
                        f"backward, fp64, {t_total:.1f} s"),
                seconds=t_total)


def parity_rows(w, causal, r, n_random=8):
    """Sampled rows of this run's output against the oracle."""
    import numpy as np
    import torch
    import oracle
    from scaled_dot_product_fa_amd import inputs
    ids = inputs.sample_rows(w.B, w.H, w.Lq, n_random=n_random, seed=w.seed,
                             heads=range(0, w.B * w.H, max(1, w.B * w.H // 8)))
    f64 = lambda t: t.to(torch.float64).numpy()
    win = r.get("window")
    win = None if win is None else tuple(win)
    ro, rl = oracle.attention_rows(f64(r["q"]), f64(r["k"]), f64(r["v"]),
                                   ids.numpy(), causal, w.scale, window=win)
    go = f64(r["o"].cpu().reshape(-1, w.D)[ids])
    gl = r["lse"].cpu().reshape(-1)[ids].double().numpy()
    return dict(rows=int(ids.numel()),
                max_abs_o=float(np.abs(go - ro).max()),
                max_abs_lse=float(np.abs(gl - rl).max()))


def cpu_baseline(w, causal, r, budget_s=15.0):
    """The fp64 oracle on a bounded, seeded row sample of the same workload
    (same mask), throughput scaled to TFLOP/s by the same FLOP formula (per
    row: 4*D*visible keys)."""
    import numpy as np
    import torch
    import oracle
    f64 = lambda t: t.to(torch.float64).numpy()
    q, k, v = f64(r["q"]), f64(r["k"]), f64(r["v"])
    win = r.get("window")
    win = None if win is None else tuple(win)
    g = np.random.default_rng(w.seed)
    total_rows = w.B * w.H * w.Lq

    def run(n):
        ids = np.sort(g.choice(total_rows, size=n, replace=False))
        i = ids % w.Lq
        lo = np.zeros(n, dtype=np.int64)
        hi = np.full(n, w.Lk - 1, dtype=np.int64)
        if causal:
            hi = np.minimum(hi, i)
        if win is not None and win[0] >= 0:
            lo = np.maximum(lo, i - win[0])
        if win is not None and win[1] >= 0:
            hi = np.minimum(hi, i + win[1])
        fl = float((4.0 * np.maximum(hi - lo + 1, 0) * w.D).sum())
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, ids, causal, w.scale, window=win)
        return fl, time.perf_counter() - t0

    pilot = 2048
    fl, dt = run(pilot)
    n = int(min(total_rows, max(pilot, pilot * budget_s / max(dt, 1e-3))))
    fl, dt = run(n)
    return dict(value=fl / dt / 1e12, unit="TFLOP/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=(f"{n} seeded query rows of {workload_desc(w, causal)} "
                        f"(all visible keys per row), fp64, {dt:.1f} s"),
                seconds=dt)


def traffic(kernel_name, workload, src=KERNEL_SRC):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a plain copy of known size) from the committed
    rocprofv3 summary for this kernel and workload, if it was taken on the
    current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(f"{kernel_name} {workload}")
    if not rec or rec.get("source_sha") != kernel_source_sha(src):
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="mid")
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time fa_bwd (gradients) instead of the forward")
    ap.add_argument("--layout", choices=("bhld", "blhd"), default="bhld",
                    help="forward inputs in [B,H,L,D] (default) or in "
                         "[B,L,H,D] buffers (strided views, fa_fwd_ex)")
    ap.add_argument("--window", default=None, metavar="LEFT,RIGHT",
                    help="forward with a local window (fa_fwd_ex); -1 = no "
                         "bound on that side")
    ap.add_argument("--secondary", action="store_true",
                    help="also time the 16K non-causal forward (the other "
                         "shape the metric names); off by default so that a "
                         "profile of the default command sees one workload")
    ap.add_argument("--no-secondary", action="store_true",
                    help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling "
                         "HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU "
              "path (the forward shards over heads with no exchange; see the "
              "design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_fa_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                          "launches": max(1, args.steps)}), flush=True)
        return

    w = inputs.CONFIGS[args.workload]
    causal = bool(args.causal)
    if args.backward:
        main_backward(args, w, causal)
        return
    window = None
    if args.window is not None:
        wl, wr = (int(x) for x in args.window.split(","))
        window = (wl, wr)
    r = time_forward(w, causal, args.steps, args.warmup, args.layout, window)
    tflops = r["flops"] / (r["wall_ms"] * 1e-3) / 1e12
    k_tflops = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    log(f"bench: wall {r['wall_ms']:.4f} ms/step, kernel {r['kernel_ms']:.4f} "
        f"ms/launch, {k_tflops:.1f} TFLOP/s")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else w.dtype,
        "data": "synthetic",
        "config": {"workload": workload_desc(w, causal)
                   + ("" if args.layout == "bhld" and window is None
                      else f" {args.layout} window={window}"), "B": w.B, "H": w.H,
                   "Lq": w.Lq, "Lk": w.Lk, "D": w.D, "causal": causal,
                   "scale": w.scale, "io_dtype": w.dtype,
                   "kernel": r["kernel"]},
        "pct_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbps": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(k_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic(r["kernel"], workload_desc(w, causal)),
            "kernel": r["kernel"],
            "flops_per_launch": r["flops"],
            "kernel_ms": round(r["kernel_ms"], 5),
        },
    }
    log("bench: parity rows vs oracle ...")
    out["parity"] = parity_rows(w, causal, r)
    log(f"bench: parity {out['parity']}")
    if args.secondary and args.workload == "mid":
        w2 = inputs.CONFIGS["long"]
        r2 = time_forward(w2, False, max(5, args.steps // 8),
                          max(2, args.warmup // 2))
        t2 = r2["flops"] / (r2["kernel_ms"] * 1e-3) / 1e12
        out["secondary"] = {"workload": workload_desc(w2, False),
                            "kernel": r2["kernel"],
                            "kernel_ms": round(r2["kernel_ms"], 4),
                            "tflops": round(t2, 2),
                            "frac": round(t2 / PEAK_BF16_TFLOPS, 4)}
        log(f"bench: secondary {out['secondary']}")
        del r2
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle on a row sample) ...")
        out["cpu_baseline"] = cpu_baseline(w, causal, r)
        log(f"bench: cpu baseline {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


def main_backward(args, w, causal):
    steps = args.steps if args.steps != 200 else 40
    warmup = args.warmup if args.warmup != 50 else 10
    window = None
    if args.window is not None:
        wl, wr = (int(x) for x in args.window.split(","))
        window = (wl, wr)
    r = time_backward(w, causal, steps, warmup, args.layout, window)
    tflops = r["flops"] / (r["wall_ms"] * 1e-3) / 1e12
    k_tflops = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    log(f"bench: backward wall {r['wall_ms']:.4f} ms/step, kernels "
        f"{r['kernel_ms']:.4f} ms/call, {k_tflops:.1f} TFLOP/s")
    out = {
        "metric": "attention bwd TFLOP/s (algorithmic 2.5x forward flops) and % "
                  "of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else w.dtype,
        "data": "synthetic",
        "config": {"workload": workload_desc(w, causal) + " backward"
                   + ("" if args.layout == "bhld" and window is None
                      else f" {args.layout} window={window}"), "B": w.B,
                   "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "D": w.D, "causal": causal,
                   "scale": w.scale, "io_dtype": w.dtype, "kernel": r["kernel"]},
        "pct_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(k_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic(r["kernel"], workload_desc(w, causal) + " backward",
                               BWD_KERNEL_SRC),
            "kernel": "fa_bwd call: delta, " + r["kernel"] + " (dK/dV), dQ",
            "flops_per_launch": r["flops"],
            "kernel_ms": round(r["kernel_ms"], 5),
        },
    }
    log("bench: backward parity (one head vs oracle) ...")
    out["parity"] = parity_bwd(w, causal, r)
    log(f"bench: parity {out['parity']}")
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle backward on whole heads) ...")
        out["cpu_baseline"] = cpu_baseline_bwd(w, causal, r)
        log(f"bench: cpu baseline {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
