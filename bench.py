"""Attention forward (and, with --backward, backward) throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mid]
    python bench.py --backward [--workload mid] [--causal]

One step is one fa_fwd call (the whole forward: Q load, K/V stream, QK^T,
masking, online softmax, PV, epilogue) over the workload's synthetic inputs,
already resident in HBM.  FLOPs per step = 4*B*H*Lq*Lk*D (halved when
causal).  Prints one JSON line.

Per shape the run is:
  1. settle: untimed launches for --settle seconds (default 2), so that the
     graphics clock reaches the value it holds under this load (the first
     launches on a fresh GPU run at a lower clock); stated in the line;
  2. W untimed warm-up steps;
  3. exactly K timed steps between two device synchronisations -- the line's
     `value` and `ms_per_step`; HIP events recorded on the launch stream give
     the kernel's average duration (`roofline.kernel_ms`);
  4. `sustained`: --trials (default 5) further timed runs of at least
     --trial-ms (default 200) ms each, HIP events around each; median and
     minimum per-launch time.
The graphics clock is sampled in-process (amdsmi, no child process) and
reported for steps 3 and 4 with the peak that clock allows.  The sampler
(amdsmi's initialisation and its thread) starts before step 1: started
just before step 3, the launches of the next few tens of milliseconds ran
up to 20% slower, enough to move the line of a 140 us kernel by 4-6%.

The metric names two shapes, D=128 N=4096 and N=16384, non-causal: the line's
`value` is the first (the mid workload), and `secondary` carries the same
measurement, roofline and sampled parity for the second (the 16K workload)
unless --no-secondary is given.

Extra fields: ``roofline`` (MFMA-bound; achieved TFLOP/s of the kernel vs the
published 2.5 PFLOP/s dense bf16 peak, and HBM traffic from the committed
rocprofv3 counter summary when it matches the current kernel source),
``cpu_baseline`` (the fp64 CPU oracle timed on the host cores: every row of
the mid workload fits its ~15 s budget; larger workloads use a seeded row
sample) and ``parity`` (every row the CPU baseline computed, compared with
this run's GPU output).

With --curve the run only times the forward over sequence lengths 512 to
16384 at a fixed 16384 tokens and model width 2048 (D = 64 and 128, both
masks) and prints one JSON line with every point.

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
# The figures the source pages give for this forward, all on another machine
# (context for the line, never its baseline: vs_baseline stays null).  The
# FlashAttention-2 forward article's benchmark section measures its Triton
# kernel on an A100 SXM over a sequence-length sweep at fixed batch, heads
# and head size, fp16.
PAGES_CONTEXT = {
    "hardware": "NVIDIA A100 SXM (dense fp16 tensor peak 312 TFLOP/s)",
    "source": "FlashAttention-2 forward article, benchmark section",
    "triton_fa2_fwd_tflops_at_N16384": 190,
    "torch_sdpa_fwd_tflops_at_N16384": "180-190",
    "materialised_attention_tflops": "3-4, flat in N",
    "note": "another machine and workload mix: context only",
}
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


class ClockSampler:
    """Samples the GPU's graphics clock (MHz) from a background thread of
    this process through the amdsmi library (no child process).  Reports
    null fields where amdsmi or the device is not available."""

    def __init__(self, period_s=0.005):
        self.period = period_s
        self.samples = []
        self.handle = None
        self.source = None
        self._stop = None
        self._thread = None
        self.recording = False   # samples are kept only while True
        try:
            import amdsmi
            import torch
            pr = torch.cuda.get_device_properties(0)
            bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handle_from_bdf(bdf)
            self.read()
            self.source = f"amdsmi gfx clock of {bdf}"
        except Exception as e:  # noqa: BLE001 -- best effort, reported as null
            self.handle = None
            self.source = f"unavailable ({type(e).__name__})"

    def read(self):
        info = self.amdsmi.amdsmi_get_clock_info(self.handle, self.amdsmi.AmdSmiClkType.SYS)
        return float(info["clk"])

    def __enter__(self):
        import threading
        if self.handle is None:
            return self
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    x = self.read()
                    if self.recording:
                        self.samples.append(x)
                except Exception:  # noqa: BLE001
                    pass
                self._stop.wait(self.period)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self, cus):
        if not self.samples:
            return {"mhz_mean": None, "source": self.source}
        a = sorted(self.samples)
        mean = sum(a) / len(a)
        return {"mhz_mean": round(mean, 1), "mhz_min": a[0], "mhz_max": a[-1],
                "samples": len(a), "source": self.source,
                # dense bf16 MFMA: 4096 flop per clock per CU
                "peak_tflops_at_mean_clock": round(cus * mean * 1e6 * 4096 / 1e12, 1)}


def measure(launch, stream, steps, warmup, settle_s, trials, trial_ms):
    """Settle, warm up, time exactly `steps` launches, then `trials`
    sustained runs of at least `trial_ms` ms each.  Returns timings (ms per
    launch) and the clock summary of the timed launches."""
    clock = ClockSampler()
    with clock:
        return _measure(launch, stream, steps, warmup, settle_s, trials, trial_ms, clock)


def _measure(launch, stream, steps, warmup, settle_s, trials, trial_ms, clock):
    import torch
    dev = torch.device("cuda:0")
    n_settle = 0
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            launch()
        n_settle += 8
        torch.cuda.synchronize(dev)
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    clock.recording = True
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        launch()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    kernel_ms = ev0.elapsed_time(ev1) / steps
    per_trial = max(steps, int(math.ceil(trial_ms / max(kernel_ms, 1e-3))))
    trial_ms_list = []
    for _ in range(trials):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(per_trial):
            launch()
        b.record(stream)
        torch.cuda.synchronize(dev)
        trial_ms_list.append(a.elapsed_time(b) / per_trial)
    clock.recording = False
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    srt = sorted(trial_ms_list)
    return dict(wall_ms=(t1 - t0) * 1e3 / steps, kernel_ms=kernel_ms,
                settle={"seconds": settle_s, "launches": n_settle},
                sustained={"trials": trials, "launches_per_trial": per_trial,
                           "kernel_ms_median": srt[len(srt) // 2] if srt else None,
                           "kernel_ms_min": srt[0] if srt else None,
                           "kernel_ms_all": [round(x, 5) for x in trial_ms_list]},
                clock=clock.summary(cus), cus=cus)


def time_forward(w, causal, steps, warmup, layout="bhld", window=None, settle_s=2.0,
                 trials=5, trial_ms=200.0):
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
    log(f"bench: {workload_desc(w, causal)} kernel={name} settle={settle_s}s "
        f"warmup={warmup} steps={steps} trials={trials}x{trial_ms:.0f}ms")

    def launch():
        fa.forward(dq, dk, dv, causal=causal, scale=w.scale, out=o, lse=lse,
                   stream=stream, window=window)
    r = measure(launch, stream, steps, warmup, settle_s, trials, trial_ms)
    r.update(flops=flops, bytes=w.io_bytes(), kernel=name,
             q=q, k=k, v=v, o=o.contiguous(), lse=lse, window=window)
    return r


def time_backward(w, causal, steps, warmup, layout="bhld", window=None, settle_s=2.0,
                  trials=5, trial_ms=200.0):
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
    log(f"bench: backward {workload_desc(w, causal)} kernel={name} settle={settle_s}s "
        f"warmup={warmup} steps={steps}")

    general = layout != "bhld" or window is not None
    if general:
        name = f"{name} via fa_bwd_ex ({layout}, window {window})"
        flops = 10.0 * w.B * w.H * w.D * visible_pairs(w.Lq, w.Lk, causal, window)
    else:
        flops = 2.5 * w.flops(causal)

    def launch():
        fa.backward(dq_, dk_, dv_, o, lse, dg, causal=causal, scale=w.scale,
                    dq=gq, dk=gk, dv=gv, delta=delta, stream=stream, window=window)
    r = measure(launch, stream, steps, warmup, settle_s, trials, trial_ms)
    r.update(flops=flops, kernel=name, window=window,
             q=q, k=k, v=v, g=g, dq=gq, dk=gk, dv=gv)
    return r


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


def _row_limits(w, ids, causal, win):
    """Visible key range [lo, hi] of each flat row id (the keep rule)."""
    import numpy as np
    i = ids % w.Lq
    lo = np.zeros(len(ids), dtype=np.int64)
    hi = np.full(len(ids), w.Lk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if win is not None and win[0] >= 0:
        lo = np.maximum(lo, i - win[0])
    if win is not None and win[1] >= 0:
        hi = np.minimum(hi, i + win[1])
    return lo, hi


def compare_rows(w, r, ids, ro, rl):
    """GPU output rows `ids` (flat (b*H + h)*Lq + i) against oracle rows."""
    import numpy as np
    import torch
    go = r["o"].cpu().reshape(-1, w.D)[torch.from_numpy(ids)].to(torch.float64).numpy()
    gl = r["lse"].cpu().reshape(-1)[torch.from_numpy(ids)].double().numpy()
    d = np.abs(go - ro)
    tol = 1e-5 if w.dtype == "f32" else 2e-2
    return dict(rows=int(len(ids)), of_rows=w.B * w.H * w.Lq,
                max_abs_o=float(d.max()), max_abs_lse=float(np.abs(gl - rl).max()),
                o_over_tol=int((d > tol).sum()), tol_o=tol, tol_lse=1e-3)


def parity_sampled(w, causal, r, n_random=64):
    """Sampled rows (all heads: tile boundaries, the middle, the last rows,
    seeded random rows) of this run's output against the oracle."""
    import torch
    import oracle
    from scaled_dot_product_fa_amd import inputs
    ids = inputs.sample_rows(w.B, w.H, w.Lq, n_random=n_random, seed=w.seed).numpy()
    f64 = lambda t: t.to(torch.float64).numpy()
    win = r.get("window")
    win = None if win is None else tuple(win)
    ro, rl = oracle.attention_rows(f64(r["q"]), f64(r["k"]), f64(r["v"]), ids,
                                   causal, w.scale, window=win)
    return compare_rows(w, r, ids, ro, rl)


def cpu_baseline(w, causal, r, budget_s=15.0):
    """The fp64 oracle on the host cores over the same workload (same mask):
    every row when the whole tensor fits about twice the budget (the mid
    workload does), else a seeded row sample sized to the budget.  Throughput
    is scaled to TFLOP/s by the same FLOP formula (per row: 4*D*visible
    keys).  Returns (baseline entry, row ids, oracle O rows, oracle LSE
    rows) so that parity can compare the very rows computed here."""
    import numpy as np
    import torch
    import oracle
    f64 = lambda t: t.to(torch.float64).numpy()
    q, k, v = f64(r["q"]), f64(r["k"]), f64(r["v"])
    win = r.get("window")
    win = None if win is None else tuple(win)
    g = np.random.default_rng(w.seed)
    total_rows = w.B * w.H * w.Lq

    def run(ids):
        lo, hi = _row_limits(w, ids, causal, win)
        fl = float((4.0 * np.maximum(hi - lo + 1, 0) * w.D).sum())
        t0 = time.perf_counter()
        ro, rl = oracle.attention_rows(q, k, v, ids, causal, w.scale, window=win)
        return fl, time.perf_counter() - t0, ro, rl

    pilot = np.sort(g.choice(total_rows, size=min(2048, total_rows), replace=False))
    fl, dt, _, _ = run(pilot)
    est_all = dt * total_rows / len(pilot)
    if est_all <= 2.0 * budget_s:
        ids = np.arange(total_rows, dtype=np.int64)
        what = f"all {total_rows} query rows"
    else:
        n = int(min(total_rows, max(len(pilot), len(pilot) * budget_s / max(dt, 1e-3))))
        ids = np.sort(g.choice(total_rows, size=n, replace=False))
        what = f"{n} seeded query rows (of {total_rows})"
    fl, dt, ro, rl = run(ids)
    entry = dict(value=fl / dt / 1e12, unit="TFLOP/s",
                 cores=oracle.num_threads(), kind="oracle",
                 sample=(f"{what} of {workload_desc(w, causal)} "
                         f"(all visible keys per row), fp64, {dt:.1f} s"),
                 seconds=dt)
    return entry, ids, ro, rl


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


def forward_entry(w, causal, r, layout="bhld", window=None):
    """The measured numbers of one forward shape: throughput, roofline,
    sustained trials and clock."""
    tflops = r["flops"] / (r["wall_ms"] * 1e-3) / 1e12
    k_tflops = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    sus = dict(r["sustained"])
    if sus.get("kernel_ms_median"):
        sus["tflops_median"] = round(r["flops"] / (sus["kernel_ms_median"] * 1e-3) / 1e12, 2)
        sus["frac_median"] = round(sus["tflops_median"] / PEAK_BF16_TFLOPS, 4)
    clock = dict(r["clock"])
    if clock.get("peak_tflops_at_mean_clock") and sus.get("tflops_median"):
        clock["frac_of_peak_at_mean_clock"] = round(
            sus["tflops_median"] / clock["peak_tflops_at_mean_clock"], 4)
    return {
        "workload": workload_desc(w, causal)
        + ("" if layout == "bhld" and window is None else f" {layout} window={window}"),
        "kernel": r["kernel"],
        "tflops": round(tflops, 2),
        "ms_per_step": round(r["wall_ms"], 5),
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
        "hbm_gbps": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 1),
        "settle": r["settle"],
        "sustained": sus,
        "clock": clock,
    }


CURVE_N = (512, 1024, 2048, 4096, 8192, 16384)


def seqlen_curve(settle_s=0.5, steps=40, warmup=10):
    """Forward TFLOP/s against sequence length at a fixed token count: for
    N = 512 ... 16384, B = 16384 / N sequences of N tokens, model width 2048
    (H = 2048 / D heads), D = 64 and 128, non-causal and causal, bf16, iid
    N(0, 1) inputs.  Per point: settling launches, a warm-up, then `steps`
    launches between HIP events.  One JSON line with every point."""
    import torch
    import scaled_dot_product_fa_amd as fa
    from scaled_dot_product_fa_amd import inputs
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    points = []
    for D in (128, 64):
        H = 2048 // D
        for causal in (False, True):
            for N in CURVE_N:
                B = 16384 // N
                w = inputs.Workload(f"curve{N}", B, H, N, N, D, "bf16",
                                    1.0 / math.sqrt(D), 11, ("noncausal", "causal"))
                q, k, v = (t.to(dev) for t in inputs.workload_inputs(w))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
                name = fa.fa_kernel_name(B, H, N, N, D, int(causal), w.scale,
                                         fa.dtype_code(q.dtype))

                def launch():
                    fa.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse,
                               stream=stream)
                r = measure(launch, stream, steps, warmup, settle_s, 0, 0.0)
                tf = w.flops(causal) / (r["kernel_ms"] * 1e-3) / 1e12
                pt = {"D": D, "causal": causal, "N": N, "B": B, "H": H, "kernel": name,
                      "kernel_ms": round(r["kernel_ms"], 5), "tflops": round(tf, 1),
                      "frac": round(tf / 2500.0, 4), "mhz_mean": r["clock"].get("mhz_mean")}
                points.append(pt)
                log(f"curve: D={D} {'causal' if causal else 'non-causal'} N={N} B={B} "
                    f"H={H} {name}: {r['kernel_ms'] * 1e3:.1f} us, {tf:.1f} TFLOP/s, "
                    f"clock {pt['mhz_mean']} MHz")
                del q, k, v, o, lse
    print(json.dumps({"metric": "attention fwd TFLOP/s vs sequence length "
                      "(16384 tokens, width 2048, bf16)", "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": steps, "warmup": warmup, "settle_s": settle_s,
                      "data": "synthetic", "points": points}), flush=True)


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
    ap.add_argument("--settle", type=float, default=2.0, metavar="SECONDS",
                    help="untimed launches before the warm-up, so the clock "
                         "settles (default 2 s)")
    ap.add_argument("--trials", type=int, default=5,
                    help="sustained timed runs after the K steps (default 5)")
    ap.add_argument("--trial-ms", type=float, default=200.0,
                    help="minimum length of each sustained run (default 200 ms)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 16K non-causal forward (the metric's second "
                         "shape), which runs by default after the mid workload")
    ap.add_argument("--secondary", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--curve", action="store_true",
                    help="only time the forward over sequence lengths 512..16384 "
                         "at 16384 tokens and width 2048 (D=64 and 128, both "
                         "masks), then exit")
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

    if args.curve:
        seqlen_curve()
        return

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
    r = time_forward(w, causal, args.steps, args.warmup, args.layout, window,
                     args.settle, args.trials, args.trial_ms)
    ent = forward_entry(w, causal, r, args.layout, window)
    log(f"bench: wall {r['wall_ms']:.4f} ms/step, kernel {r['kernel_ms']:.4f} "
        f"ms/launch, {ent['roofline']['achieved']:.1f} TFLOP/s; sustained "
        f"{ent['sustained']}; clock {ent['clock']}")

    out = {
        "metric": METRIC,
        "value": ent["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ent["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else w.dtype,
        "data": "synthetic",
        "config": {"workload": ent["workload"], "B": w.B, "H": w.H,
                   "Lq": w.Lq, "Lk": w.Lk, "D": w.D, "causal": causal,
                   "scale": w.scale, "io_dtype": w.dtype,
                   "kernel": r["kernel"]},
        "pct_peak": round(100.0 * ent["tflops"] / PEAK_BF16_TFLOPS, 2),
        "hbm_gbps": ent["hbm_gbps"],
        "roofline": ent["roofline"],
        "settle": ent["settle"],
        "sustained": ent["sustained"],
        "clock": ent["clock"],
        "context": PAGES_CONTEXT,
    }
    # the CPU baseline first: parity then compares every row it computed
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (the oracle on the host cores) ...")
        base, ids, ro, rl = cpu_baseline(w, causal, r)
        out["cpu_baseline"] = base
        log(f"bench: cpu baseline {base}")
        out["parity"] = compare_rows(w, r, ids, ro, rl)
        del ro, rl
    else:
        out["parity"] = parity_sampled(w, causal, r)
    log(f"bench: parity {out['parity']}")
    del r
    if not args.no_secondary and args.workload == "mid" and not causal \
            and args.layout == "bhld" and window is None:
        w2 = inputs.CONFIGS["long"]
        torch.cuda.empty_cache()
        r2 = time_forward(w2, False, args.steps, args.warmup, settle_s=args.settle,
                          trials=args.trials, trial_ms=args.trial_ms)
        sec = forward_entry(w2, False, r2)
        log("bench: secondary parity (sampled rows) ...")
        sec["parity"] = parity_sampled(w2, False, r2)
        out["secondary"] = sec
        log(f"bench: secondary {sec}")
        del r2
        out["metric_shapes"] = {
            "N=4096": {"tflops": out["value"], "frac": out["roofline"]["frac"],
                       "frac_sustained": out["sustained"].get("frac_median")},
            "N=16384": {"tflops": sec["tflops"], "frac": sec["roofline"]["frac"],
                        "frac_sustained": sec["sustained"].get("frac_median")},
        }
    print(json.dumps(out), flush=True)


def main_backward(args, w, causal):
    steps = args.steps if args.steps != 200 else 40
    warmup = args.warmup if args.warmup != 50 else 10
    window = None
    if args.window is not None:
        wl, wr = (int(x) for x in args.window.split(","))
        window = (wl, wr)
    r = time_backward(w, causal, steps, warmup, args.layout, window, args.settle,
                      args.trials, args.trial_ms)
    tflops = r["flops"] / (r["wall_ms"] * 1e-3) / 1e12
    k_tflops = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    log(f"bench: backward wall {r['wall_ms']:.4f} ms/step, kernels "
        f"{r['kernel_ms']:.4f} ms/call, {k_tflops:.1f} TFLOP/s")
    sus = dict(r["sustained"])
    if sus.get("kernel_ms_median"):
        sus["tflops_median"] = round(r["flops"] / (sus["kernel_ms_median"] * 1e-3) / 1e12, 2)
        sus["frac_median"] = round(sus["tflops_median"] / PEAK_BF16_TFLOPS, 4)
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
        "settle": r["settle"],
        "sustained": sus,
        "clock": r["clock"],
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
