"""The forward profile summaries name the code that ran (CPU only).

Each forward summary under profiles/ that records a kernel symbol is titled
with the label fa_kernel_name gives its workload.  The label's family, I/O
type, head dimension, mask and key-tile size must agree with the template
arguments of the symbol rocprofv3 recorded, and profiles/traffic.json must
key its HBM figure by that label and workload.
"""
import glob
import json
import os
import re

import pytest

import scaled_dot_product_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAMILY = {"pp": "fa_fwd_mfma_pp_kernel", "ppp": "fa_fwd_mfma_pers_kernel",
          "pipe": "fa_fwd_mfma_dma_kernel", "reg": "fa_fwd_mfma_kernel"}


def summaries():
    out = []
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "fa_fwd_mfma_*.txt"))):
        lines = open(p).read().splitlines()
        sym = [ln[len("kernel symbol: "):] for ln in lines if ln.startswith("kernel symbol: ")]
        if sym:
            out.append((os.path.basename(p), lines[0], sym[0]))
    return out


def test_headline_summaries_exist():
    names = [s[0] for s in summaries()]
    assert "fa_fwd_mfma_bf16_d128_pp8w_bn64_mid_noncausal.txt" in names
    assert "fa_fwd_mfma_bf16_d128_pp8w_bn64_long_noncausal.txt" in names


@pytest.mark.parametrize("fname,title,symbol", summaries(), ids=[s[0] for s in summaries()])
def test_label_matches_symbol_and_workload(fname, title, symbol):
    label, rest = title.split(" -- ", 1)
    assert fname.startswith(label + "_")
    m = re.match(r"fa_fwd_mfma_(bf16|f16)_d(\d+)(_causal)?_(ppp|pp|pipe|reg)(\d+)w(\d+q)?_bn(\d+)", label)
    assert m, label
    dt, D, causal, fam, nw, qb, bn = m.groups()
    # the template: <Ops, D, CAUSAL, BN, GEN, WIN> for pp, <Ops, D, BN> for ppp
    assert FAMILY[fam] + "<" in symbol, (fam, symbol)
    targs = symbol.split("<", 1)[1].split(">(")[0]
    args = [a.strip() for a in re.sub(r"fa::\(anonymous namespace\)::", "", targs).split(",")]
    assert args[0] == {"bf16": "Bf16Ops", "f16": "F16Ops"}[dt]
    assert args[1] == D
    if fam == "pp":
        assert args[2] == ("true" if causal else "false")
        assert args[3] == bn
        assert args[4:] == ["false", "false"]        # contiguous, no window
    elif fam == "ppp":
        assert not causal and args[2] == bn
    # the workload in the title gets this label from fa_kernel_name
    w = re.match(r"(\S+) B=(\d+) H=(\d+) Lq=(\d+) Lk=(\d+) D=(\d+) (\S+) (\S+)", rest.split(", MI355X")[0])
    name, B, H, Lq, Lk, Dw, wdt, mode = w.groups()
    assert int(Dw) == int(D) and wdt == dt and (mode == "causal") == bool(causal)
    scale = 1.0 / float(Dw) ** 0.5
    assert fa.fa_kernel_name(int(B), int(H), int(Lq), int(Lk), int(Dw), int(mode == "causal"),
                             scale, {"bf16": 2, "f16": 1}[dt]) == label


def test_traffic_is_keyed_by_label_and_workload():
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for fname, title, _ in summaries():
        label, rest = title.split(" -- ", 1)
        key = f"{label} {rest.split(', MI355X')[0]}"
        assert key in t, key
        rec = t[key]
        assert rec["summary"] == fname
        assert rec["bytes_per_launch"] > 0 and rec["algorithmic_bytes"] > 0
        assert 0.9 < rec["bytes_per_launch"] / rec["algorithmic_bytes"] < 3.0
