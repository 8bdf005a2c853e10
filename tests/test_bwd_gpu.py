"""GPU parity of the backward: fa_bwd (through the C ABI) against the oracle's
fp64 chain-rule gradients.

Gradients are far from unit scale (for N(0, 1) inputs dV_j is about
sqrt(e / Lq)), so the stated max-abs bars (2e-2 for bf16/fp16 I/O, 1e-5 for
fp32) are applied to the error divided by the largest reference magnitude of
that tensor: max|g - ref| <= tol * max|ref|.  The bf16/fp16 kernels round the
probabilities and ds to the I/O type before they multiply tensors (relative
error 2^-8 for bf16, 2^-11 for fp16), which gives a normalised error of a few
1e-3 at most; a wrong term (a dropped delta, a missing scale, a transposed
operand) gives an error of order one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to64(t):
    return t.to(torch.float64).numpy()


def run_gpu(q, k, v, g, causal, scale):
    dev = torch.device("cuda:0")
    q, k, v, g = (t.to(dev) for t in (q, k, v, g))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    delta = torch.empty(lse.shape, device=dev, dtype=torch.float32)
    dq, dk, dv = fa.backward(q, k, v, o, lse, g, causal=causal, scale=scale,
                             delta=delta)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), delta.cpu()


def norm_err(a, ref, scale_ref=None):
    """max|a - ref| / max|ref|.  A reference that is exactly zero (Lk = 1
    gives dq = dk = 0: p = 1 and ds = p (dp - delta) = 0) is measured against
    ``scale_ref``, the largest |dV| of the same problem, instead: the GPU
    leaves a rounding residue there (delta uses o rounded to the I/O type)."""
    denom = np.abs(ref).max()
    if denom == 0.0 and scale_ref is not None:
        denom = scale_ref
    return float(np.abs(to64(a) - ref).max() / max(denom, 1e-30))


def check(B, H, Lq, Lk, D, dt, causal, scale=None, seed=0, label=""):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed)
    g = inputs.make_dout(B, H, Lq, D, dt, seed)
    name = fa.fa_bwd_kernel_name(B, H, Lq, Lk, D, int(causal), scale,
                                 fa.dtype_code(q.dtype))
    say(f"[bwd] {label} B={B} H={H} Lq={Lq} Lk={Lk} D={D} {dt} "
        f"causal={causal} scale={scale:.5g} kernel={name}")
    dq, dk, dv, delta = run_gpu(q, k, v, g, causal, scale)
    rq, rk, rv, rd = oracle.attention_bwd(to64(q), to64(k), to64(v), to64(g),
                                          causal, scale, with_delta=True)
    sv = float(np.abs(rv).max())
    errs = {n: norm_err(a, r, sv) for n, a, r in (("dq", dq, rq), ("dk", dk, rk),
                                                 ("dv", dv, rv), ("delta", delta, rd))}
    say("[bwd]   " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for t in (dq, dk, dv, delta):
        assert torch.isfinite(t.float()).all()
    for n, e in errs.items():
        assert e <= TOL[dt], (n, e)
    return errs


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_tiny_workload(causal):
    w = inputs.CONFIGS["tiny"]
    check(w.B, w.H, w.Lq, w.Lk, w.D, w.dtype, causal, w.scale, w.seed, "tiny")


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_small_workload(causal):
    w = inputs.CONFIGS["small"]
    check(w.B, w.H, w.Lq, w.Lk, w.D, w.dtype, causal, w.scale, w.seed, "small")


RAGGED = [(1, 2, 200, 333, 128, "bf16"), (2, 1, 77, 45, 64, "f16"),
          (1, 1, 300, 100, 64, "bf16"), (1, 1, 1, 1, 128, "bf16"),
          (1, 2, 1, 257, 64, "f16"), (1, 1, 257, 1, 128, "bf16"),
          (1, 1, 130, 190, 128, "f32"), (1, 3, 95, 64, 64, "f32")]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_ragged(shape, causal):
    B, H, Lq, Lk, D, dt = shape
    check(B, H, Lq, Lk, D, dt, causal, seed=Lq + Lk + D, label="ragged")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
def test_other_scales(scale):
    check(1, 2, 96, 150, 64, "bf16", True, scale=scale, seed=5, label="scale")


def test_deterministic():
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs.make_qkv(1, 4, 333, 300, 128, "bf16", 9))
    g = inputs.make_dout(1, 4, 333, 128, "bf16", 9).to(dev)
    o, lse = fa.forward(q, k, v, causal=True)
    a = fa.backward(q, k, v, o, lse, g, causal=True)
    b = fa.backward(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# MFMA tile edges: 128-key / 128-query workgroup blocks, 32-row query tiles
# (dK/dV kernel) and 64-key tiles (dQ kernel), ragged on both sides.
EDGES = [(1, 1, 31, 33), (1, 1, 32, 32), (1, 1, 33, 31), (1, 1, 127, 129),
         (1, 1, 128, 128), (1, 1, 129, 127), (1, 2, 255, 257), (1, 1, 64, 300),
         (1, 1, 300, 64), (2, 1, 513, 450)]


@pytest.mark.parametrize("lens", EDGES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("D,dt", [(128, "bf16"), (64, "f16")], ids=["d128bf16", "d64f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_tile_edges(lens, D, dt, causal):
    B, H, Lq, Lk = lens
    check(B, H, Lq, Lk, D, dt, causal, seed=3 * Lq + Lk, label="edges")


def test_matches_valu_path(monkeypatch):
    """The MFMA and vector-ALU backward agree on the same inputs (both are
    also checked against the oracle above)."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs.make_qkv(2, 2, 300, 260, 128, "bf16", 21))
    g = inputs.make_dout(2, 2, 300, 128, "bf16", 21).to(dev)
    o, lse = fa.forward(q, k, v, causal=True)
    a = fa.backward(q, k, v, o, lse, g, causal=True)
    monkeypatch.setenv("FA_TILE", "valu")
    assert fa.fa_bwd_kernel_name(2, 2, 300, 260, 128, 1, 0.1, 2).startswith("fa_bwd_valu")
    b = fa.backward(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        ref = y.float().abs().max().item()
        assert (x.float() - y.float()).abs().max().item() <= 2e-2 * ref


# Full-size workloads: the whole backward runs at full size, and the
# gradients of sampled heads are compared with the oracle run on those heads
# alone (heads are independent).
@pytest.mark.parametrize("name,mode,heads", [
    ("mid", "noncausal", [(0, 0), (3, 15)]),
    ("mid", "causal", [(1, 7)]),
    ("long", "causal", [(0, 31)]),
    ("xattn", "noncausal", [(0, 0), (7, 9)]),
    ("xattn_lk4000", "noncausal", [(5, 3)]),
])
def test_workload_sampled_heads(name, mode, heads):
    w = inputs.CONFIGS[name]
    causal = mode == "causal"
    q, k, v = inputs.workload_inputs(w)
    g = inputs.make_dout(w.B, w.H, w.Lq, w.D, w.dtype, w.seed)
    say(f"[bwd] {name}/{mode} B={w.B} H={w.H} Lq={w.Lq} Lk={w.Lk} D={w.D} "
        f"{w.dtype} kernel={fa.fa_bwd_kernel_name(w.B, w.H, w.Lq, w.Lk, w.D, int(causal), w.scale, fa.dtype_code(q.dtype))}")
    dq, dk, dv, _ = run_gpu(q, k, v, g, causal, w.scale)
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_bwd(to64(q[sl]), to64(k[sl]), to64(v[sl]),
                                          to64(g[sl]), causal, w.scale)
        errs = {"dq": norm_err(dq[sl], rq), "dk": norm_err(dk[sl], rk),
                "dv": norm_err(dv[sl], rv)}
        say(f"[bwd]   head ({b},{h}) " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL[w.dtype], (n, e)


# Seeded random shapes for the backward: Lq, Lk drawn from 1..600, D in
# {64, 128}, bf16/fp16/fp32, causal or not, scales from the usual 1/sqrt(D)
# to a negative one; all gradients against the oracle's.
def _random_bwd_cases(n=20, seed=77):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(g.choice([64, 128]))
        dt = str(g.choice(["bf16", "f16", "f32"], p=[0.45, 0.45, 0.1]))
        scale = float(g.choice([1.0 / math.sqrt(D), 0.05, -0.07]))
        cases.append((i, 1 + int(g.integers(0, 2)), 1 + int(g.integers(0, 2)),
                      int(g.integers(1, 601)), int(g.integers(1, 601)), D, dt,
                      bool(g.integers(0, 2)), scale))
    return cases


@pytest.mark.parametrize("case", _random_bwd_cases(), ids=lambda c: f"r{c[0]}")
def test_random_shapes_bwd(case):
    i, B, H, Lq, Lk, D, dt, causal, scale = case
    check(B, H, Lq, Lk, D, dt, causal, scale=scale, seed=500 + i, label=f"random r{i}")
