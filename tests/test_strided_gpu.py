"""GPU parity of fa_fwd_ex: strided views and the local window, against the
oracle on contiguous copies (the layout does not change the mathematics).

Tolerances as for fa_fwd: max-abs on O of 2e-2 (bf16/fp16 I/O) or 1e-5
(fp32), 1e-3 on LSE.  Rows that keep no key must give O = 0, LSE = -inf.
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

TOL_O = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def compare(o, lse, q, k, v, causal, scale, dt, window=None, label=""):
    ro, rl = oracle.attention(to64(q), to64(k), to64(v), causal, scale, window=window)
    go, gl = to64(o), lse.detach().cpu().double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), "rows without keys"
    assert np.all(go[empty] == 0)
    eo = float(np.abs(go - ro).max())
    el = float(np.abs(gl[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"[ex] {label} max|dO|={eo:.3e} max|dLSE|={el:.3e} empty_rows={int(empty.sum())}")
    assert eo <= TOL_O[dt], eo
    assert el <= 1e-3, el


def blhd(t):
    """The same values in a [B, L, H, D] buffer, viewed as [B, H, L, D]."""
    return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)


def padded(t, pad=8):
    """The same values in rows of D + pad elements (row stride D + pad)."""
    B, H, L, D = t.shape
    big = torch.zeros((B, H, L, D + pad), dtype=t.dtype)
    big[..., :D] = t
    return big.to(DEV)[..., :D]


LAYOUT_CASES = [(2, 3, 257, 300, 128, "bf16"), (1, 4, 100, 64, 64, "f16"),
                (2, 2, 64, 129, 128, "f16"), (1, 2, 130, 190, 64, "f32"),
                (4, 8, 512, 512, 128, "bf16")]


@pytest.mark.parametrize("shape", LAYOUT_CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["blhd", "padded", "mixed"])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_layouts(shape, layout, causal):
    B, H, Lq, Lk, D, dt = shape
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + 7 * Lk + D)
    if layout == "blhd":
        gq, gk, gv = blhd(q), blhd(k), blhd(v)
    elif layout == "padded":
        gq, gk, gv = padded(q), padded(k, 16), padded(v, 24)
    else:
        gq, gk, gv = blhd(q), padded(k), v.to(DEV)
    assert not gq.is_contiguous() or not gk.is_contiguous()
    o, lse = fa.forward(gq, gk, gv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    if layout == "blhd":
        assert o.stride() == gq.stride()   # the output follows q's layout
    compare(o, lse, q, k, v, causal, scale, dt, label=f"{layout} {shape} causal={causal}")


def test_packed_qkv():
    B, H, L, D = 2, 4, 300, 128
    q, k, v = inputs.make_qkv(B, H, L, L, D, "bf16", seed=11)
    packed = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().to(DEV)
    gq, gk, gv = (packed[:, :, i].transpose(1, 2) for i in range(3))   # [B, L, 3, H, D]
    o, lse = fa.forward(gq, gk, gv, causal=True)
    torch.cuda.synchronize()
    compare(o, lse, q, k, v, True, 1.0 / math.sqrt(D), "bf16", label="packed qkv")


def test_strided_output():
    B, H, L, D = 1, 2, 200, 64
    q, k, v = inputs.make_qkv(B, H, L, L, D, "f16", seed=12)
    out = torch.zeros((B, L, H, D + 8), dtype=torch.float16, device=DEV)[..., :D].transpose(1, 2)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    compare(o, lse, q, k, v, False, 1.0 / math.sqrt(D), "f16", label="strided out")


WINDOWS = [(False, (16, 16)), (True, (64, None)), (False, (0, 0)), (True, (100, None)),
           (False, (None, 37)), (False, (130, 5)), (True, (1, None)), (False, (255, 255))]


@pytest.mark.parametrize("cw", WINDOWS, ids=lambda c: f"c{int(c[0])}_{c[1][0]}_{c[1][1]}")
@pytest.mark.parametrize("shape", [(1, 2, 300, 300, 128, "bf16"), (2, 1, 257, 190, 64, "f16"),
                                   (1, 2, 160, 170, 64, "f32"), (1, 1, 513, 513, 128, "f16")],
                         ids=lambda s: "x".join(map(str, s)))
def test_windows(shape, cw):
    causal, (wl, wr) = cw
    B, H, Lq, Lk, D, dt = shape
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + Lk + (wl or 0))
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                        window=(wl, wr))
    torch.cuda.synchronize()
    win = (-1 if wl is None else wl, -1 if wr is None else wr)
    compare(o, lse, q, k, v, causal, scale, dt, window=win,
            label=f"window {win} causal={causal} {shape}")


def test_window_rows_without_keys():
    """Lq > Lk with a narrow window: later rows see no key (O = 0, LSE = -inf)."""
    B, H, Lq, Lk, D = 1, 2, 400, 100, 128
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, "bf16", seed=13)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), window=(8, 8))
    torch.cuda.synchronize()
    compare(o, lse, q, k, v, False, 1.0 / math.sqrt(D), "bf16", window=(8, 8), label="empty rows")


def test_window_valu_matches_mfma(monkeypatch):
    B, H, L, D = 1, 2, 300, 128
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, H, L, L, D, "bf16", seed=14))
    a, la = fa.forward(q, k, v, causal=True, window=(40, None))
    monkeypatch.setenv("FA_TILE", "valu")
    b, lb = fa.forward(q, k, v, causal=True, window=(40, None))
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 2e-2
    assert (la - lb).abs().max().item() <= 1e-3


def test_contiguous_ex_is_fa_fwd():
    """fa_fwd_ex with the contiguous strides and no window is fa_fwd, bit for
    bit (the same kernel)."""
    B, H, L, D = 2, 4, 1024, 128
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, H, L, L, D, "bf16", seed=15))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = [x for t in (q, k, v, o2) for x in t.stride()[:3]]
    rc = fa.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                      B, H, L, L, D, st, 1, -1, -1, 1.0 / math.sqrt(D), fa.dtype_code(q.dtype),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name,causal,window", [("mid", False, None), ("long", True, (1024, None)),
                                                ("xattn", False, (256, 256))])
def test_workload_blhd_sampled(name, causal, window):
    """Full-size workloads in the [B, L, H, D] layout (optionally windowed),
    sampled rows against the oracle."""
    w = inputs.CONFIGS[name]
    q, k, v = inputs.workload_inputs(w)
    say(f"[ex] {name} blhd causal={causal} window={window}")
    o, lse = fa.forward(blhd(q), blhd(k), blhd(v), causal=causal, scale=w.scale, window=window)
    torch.cuda.synchronize()
    ids = inputs.sample_rows(w.B, w.H, w.Lq, n_random=8, seed=w.seed,
                             heads=range(0, w.B * w.H, max(1, w.B * w.H // 8)))
    win = None if window is None else tuple(-1 if x is None else x for x in window)
    ro, rl = oracle.attention_rows(to64(q), to64(k), to64(v), ids.numpy(), causal, w.scale,
                                   window=win)
    go = to64(o.contiguous()).reshape(-1, w.D)[ids.numpy()]
    gl = lse.cpu().reshape(-1)[ids].double().numpy()
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    say(f"[ex]   rows={ids.numel()} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O[w.dtype] and el <= 1e-3


# Grids of 512+ blocks of 256 rows take the ping-pong kernel on the strided /
# windowed path; checked on sampled rows (all heads sampled by stride).
PP_CASES = [((4, 32, 1024, 1024, 128, "bf16"), False, None),
            ((4, 32, 1024, 1024, 128, "bf16"), True, None),
            ((4, 32, 1024, 1100, 64, "f16"), False, None),
            ((4, 32, 1024, 1024, 128, "bf16"), True, (64, None)),
            ((4, 32, 1024, 1024, 128, "bf16"), False, (100, 100)),
            ((4, 32, 1024, 1100, 64, "f16"), True, (300, None)),
            # rows past Lk + 16 see no key: whole workgroups skip their tiles
            ((2, 32, 2048, 512, 128, "bf16"), False, (16, 16))]


@pytest.mark.parametrize("case", PP_CASES, ids=lambda c: f"{'x'.join(map(str, c[0]))}_c{int(c[1])}_{c[2]}")
def test_pingpong_general_sampled(case):
    (B, H, Lq, Lk, D, dt), causal, window = case
    assert B * H * ((Lq + 255) // 256) >= 512
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + Lk + D + B)
    o, lse = fa.forward(blhd(q), blhd(k), blhd(v), causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    ids = inputs.sample_rows(B, H, Lq, n_random=12, seed=D, heads=range(0, B * H, 5))
    win = None if window is None else tuple(-1 if x is None else x for x in window)
    ro, rl = oracle.attention_rows(to64(q), to64(k), to64(v), ids.numpy(), causal, scale,
                                   window=win)
    go = to64(o.contiguous()).reshape(-1, D)[ids.numpy()]
    gl = lse.cpu().reshape(-1)[ids].double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty)
    assert np.all(go[empty] == 0)
    eo = float(np.abs(go - ro).max())
    el = float(np.abs(gl[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"[ex] pingpong general {case}: rows={ids.numel()} empty={int(empty.sum())} "
        f"max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O[dt] and el <= 1e-3


# The windowed ping-pong kernel with scores that climb across the keys, so
# that its stabiliser moves (one key whose probability alone would pass the
# fp16 range, then a whole tile of larger scores) while some waves have not
# yet seen a key of their window.
def test_pingpong_window_stabiliser_moves():
    B, H, L, D, dt = 1, 128, 1024, 128, "bf16"
    assert B * H * ((L + 255) // 256) >= 512
    g = torch.Generator().manual_seed(11)
    t = torch.zeros(L)
    t[96:] = 40.0
    t[200] = 200.0
    t[288:384] = 300.0
    t[384:] = 295.0
    q = (1.0 + 0.05 * torch.randn(B, H, L, D, generator=g)).to(torch.bfloat16)
    k = (t.view(1, 1, L, 1) / D + 0.02 * torch.randn(B, H, L, D, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, H, L, D, generator=g).to(torch.bfloat16)
    scale = 0.09
    o, lse = fa.forward(blhd(q), blhd(k), blhd(v), causal=True, scale=scale, window=(256, None))
    torch.cuda.synchronize()
    ids = inputs.sample_rows(B, H, L, n_random=16, seed=3, heads=range(0, B * H, 9))
    ro, rl = oracle.attention_rows(to64(q), to64(k), to64(v), ids.numpy(), True, scale,
                                   window=(256, -1))
    go = to64(o.contiguous()).reshape(-1, D)[ids.numpy()]
    gl = lse.cpu().reshape(-1)[ids].double().numpy()
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    say(f"[ex] pingpong window stabiliser: rows={ids.numel()} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    assert eo <= TOL_O[dt] and el <= 1e-3
