"""Host logic of bench.py (CPU only): the single-GPU guard, the FLOP and
byte conventions, visible-pair counts behind the windowed FLOPs, and the
rule that HBM traffic is reported only for the kernel source it was
measured on."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from scaled_dot_product_fa_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _pairs_brute(Lq, Lk, causal, window):
    n = 0
    for i in range(Lq):
        for j in range(Lk):
            keep = (not causal) or j <= i
            if window is not None:
                wl, wr = window
                keep = keep and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
            n += keep
    return n


def test_visible_pairs_closed_forms_and_brute_force():
    assert bench.visible_pairs(300, 450, False, None) == 300 * 450
    assert bench.visible_pairs(257, 257, True, None) == 257 * 258 // 2
    # top-left causal with Lq > Lk: rows past Lk see every key
    assert bench.visible_pairs(10, 4, True, None) == 1 + 2 + 3 + 4 * 7
    for Lq, Lk, causal, window in [(37, 53, True, (5, -1)), (53, 37, False, (3, 2)),
                                   (40, 40, True, (0, -1)), (17, 29, False, (-1, 4)),
                                   (9, 9, False, (100, 100))]:
        assert bench.visible_pairs(Lq, Lk, causal, window) == \
            _pairs_brute(Lq, Lk, causal, window), (Lq, Lk, causal, window)


def test_workload_flops_and_bytes_conventions():
    w = inputs.CONFIGS["mid"]
    assert w.flops(False) == 4.0 * 4 * 16 * 4096 * 4096 * 128
    assert w.flops(True) == w.flops(False) / 2
    # Q, K, V read once, O written once (bf16), LSE written once (fp32)
    assert w.io_bytes() == 2 * 4 * 16 * (2 * 4096 + 2 * 4096) * 128 + 4 * 4 * 16 * 4096
    x = inputs.CONFIGS["xattn"]
    assert x.flops(False) == 4.0 * 8 * 16 * 1024 * 4096 * 64


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of a kernel\n")
    tf = tmp_path / "traffic.json"
    key = "fa_fwd_mfma_bf16_d128 mid B=4 H=16 Lq=4096 Lk=4096 D=128 bf16 non-causal"
    tf.write_text(json.dumps({key: {"source_sha": bench.kernel_source_sha(str(src)),
                                    "bytes_per_launch": 269.7e6}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    kernel, workload = key.split(" ", 1)
    assert bench.traffic(kernel, workload, str(src)) == 269.7e6
    assert bench.traffic(kernel, workload + " causal", str(src)) is None
    src.write_text("// the kernel after an edit\n")
    assert bench.traffic(kernel, workload, str(src)) is None


def test_committed_traffic_records_are_consistent():
    t = json.load(open(bench.TRAFFIC_FILE))
    for key, rec in t.items():
        b = rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]
        assert np.isclose(b, rec["bytes_per_launch"], rtol=1e-9), key
        assert os.path.exists(os.path.join(ROOT, "profiles", rec["summary"])), key
