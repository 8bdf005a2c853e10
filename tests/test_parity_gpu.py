"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances are the ones the target states: max-abs error on O of 2e-2 for
bf16/fp16 I/O and 1e-5 for fp32 I/O, and 1e-3 on the natural-log LSE.
Every named workload, the full-size ones included, is compared element by
element over the whole output (the oracle runs head by head on the host
cores, about a minute for the 16K workload).  Extra large shapes are compared
on sampled rows (tile boundaries, the middle, the last rows and seeded random
rows), which the oracle computes one by one.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to64(t):
    return t.to(torch.float64).numpy()


def gpu_forward(q, k, v, causal, scale):
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o, lse = fa.forward(dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_full(q, k, v, causal, scale, dtype, label=""):
    say(f"[parity] {label} q{tuple(q.shape)} k{tuple(k.shape)} {dtype} "
        f"causal={causal} scale={scale:.6g} "
        f"kernel={fa.fa_kernel_name(*q.shape[:3], k.shape[2], q.shape[3], int(causal), scale, fa.dtype_code(q.dtype))}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    ro, rl = oracle.attention(to64(q), to64(k), to64(v), causal, scale)
    eo = np.abs(to64(o) - ro).max()
    el = np.abs(lse.double().numpy() - rl).max()
    say(f"[parity]   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(to64(o)).all() and np.isfinite(lse.numpy()).all()
    assert eo <= TOL_O[dtype], eo
    assert el <= TOL_LSE, el
    return o, lse


# ---------------------------------------------------------------- workloads

def check_whole(q, k, v, causal, scale, dtype, label, heads_per_chunk=4):
    """The whole output of one GPU call against the oracle, which runs a few
    heads at a time (progress printed per chunk).  Returns the worst errors
    and the count of O elements over the bar."""
    B, H, Lq, D = q.shape
    say(f"[parity] {label} B={B} H={H} Lq={Lq} Lk={k.shape[2]} D={D} {dtype} "
        f"causal={causal} whole output, kernel="
        f"{fa.fa_kernel_name(B, H, Lq, k.shape[2], D, int(causal), scale, fa.dtype_code(q.dtype))}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(lse.numpy()).all()
    qf, kf, vf = (t.reshape(B * H, 1, t.shape[2], D) for t in (q, k, v))
    of, lf = o.reshape(B * H, Lq, D), lse.reshape(B * H, Lq)
    eo = el = 0.0
    over = 0
    for h0 in range(0, B * H, heads_per_chunk):
        sl = slice(h0, min(B * H, h0 + heads_per_chunk))
        ro, rl = oracle.attention(to64(qf[sl]), to64(kf[sl]), to64(vf[sl]), causal, scale)
        d = np.abs(to64(of[sl]) - ro[:, 0])
        eo = max(eo, float(d.max()))
        over += int((d > TOL_O[dtype]).sum())
        el = max(el, float(np.abs(lf[sl].double().numpy() - rl[:, 0]).max()))
        if B * H > heads_per_chunk:
            say(f"[parity]   heads {sl.start}..{sl.stop - 1}: max|dO|={eo:.3e} "
                f"max|dLSE|={el:.3e} over={over}")
    say(f"[parity]   rows={B * H * Lq} max|dO|={eo:.3e} max|dLSE|={el:.3e} over={over}")
    return eo, el, over


def _workload_case(name, mode):
    w = inputs.CONFIGS[name]
    causal = mode == "causal"
    q, k, v = inputs.workload_inputs(w)
    if w.name == "tiny" or w.name == "small":
        check_full(q, k, v, causal, w.scale, w.dtype, f"{name}/{mode}")
        return
    eo, el, over = check_whole(q, k, v, causal, w.scale, w.dtype, f"{name}/{mode}")
    assert eo <= TOL_O[w.dtype] and over == 0, (eo, over)
    assert el <= TOL_LSE, el


WORKLOAD_CASES = [(n, m) for n, w in inputs.CONFIGS.items() for m in w.modes]


@pytest.mark.parametrize("name,mode", WORKLOAD_CASES,
                         ids=[f"{n}-{m}" for n, m in WORKLOAD_CASES])
def test_workload(name, mode):
    _workload_case(name, mode)


# A peaky bf16 workload small enough for a whole-output check: 1% of the
# keys scaled by 8, so many rows are dominated by one key whose p is not a
# power of two (the bias a denominator of unrounded p would leave is about
# 2.6e-2 here; the floor of rounding the exact O to bf16 is 1.56e-2).  Every
# bf16 kernel family: the default choice, both ping-pong tile sizes and the
# software-pipelined kernel.
PEAKY_TILES = [None, "8x1x64x2x3", "8x1x96x2x3", "8x1x64x2x2", "4x1x64x2x2"]


@pytest.mark.parametrize("tile", PEAKY_TILES, ids=[str(t) for t in PEAKY_TILES])
@pytest.mark.parametrize("causal", [False, True])
def test_peaky_whole_output(tile, causal, monkeypatch):
    if tile is not None:
        monkeypatch.setenv("FA_TILE", tile)
    B, H, L, D = 1, 16, 2048, 128
    q, k, v = inputs.make_qkv(B, H, L, L, D, "bf16", seed=11, peaky_frac=0.01,
                              peaky_factor=8.0)
    eo, el, over = check_whole(q, k, v, causal, 1.0 / math.sqrt(D), "bf16",
                               f"peaky tile={tile}", heads_per_chunk=16)
    assert eo <= 1.7e-2 and over == 0, (eo, over)
    assert el <= TOL_LSE, el


# ------------------------------------------------- ragged multi-tile shapes

RAGGED = [
    # B, H, Lq, Lk, D, dtype
    (1, 3, 333, 517, 128, "bf16"),
    (2, 2, 257, 190, 64, "f16"),
    (1, 2, 130, 77, 128, "f32"),
    (1, 1, 1, 1, 64, "bf16"),
    (1, 1, 1, 1000, 128, "bf16"),
    (1, 2, 700, 1, 64, "f16"),
    (2, 1, 64, 64, 128, "bf16"),
    (1, 1, 129, 4001, 64, "f16"),
    (1, 2, 600, 260, 128, "bf16"),   # Lq > Lk, causal rows past Lk see all
    (3, 1, 95, 97, 64, "f32"),
]


@pytest.mark.parametrize("shape", RAGGED, ids=[str(s) for s in RAGGED])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged(shape, causal):
    B, H, Lq, Lk, D, dt = shape
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=B + H + Lq + Lk + D)
    check_full(q, k, v, causal, 1.0 / math.sqrt(D), dt, "ragged")


@pytest.mark.parametrize("tile", ["4x1x64x1x0", "4x1x64x2x0", "8x1x64x2x0", "4x2x64x1x0",
                                  "8x1x64x2x2", "4x1x64x2x2", "4x2x64x1x2", "2x1x64x1x2", "1x1x64x1x2",
                                  "8x1x64x2x3", "8x1x128x2x3",
                                  "8x1x96x2x3", "valu"])
@pytest.mark.parametrize("D,dt", [(64, "bf16"), (128, "f16")])
def test_tile_variants(tile, D, dt, monkeypatch):
    if tile == "8x1x128x2x3" and D == 128:
        pytest.skip("128-key ping-pong tiles are built for D=64 only (LDS)")
    if tile == "8x1x96x2x3" and D == 64:
        pytest.skip("96-key ping-pong tiles are built for D=128 only (1.5 loads per lane at D=64)")
    monkeypatch.setenv("FA_TILE", tile)
    for causal in (False, True):
        q, k, v = inputs.make_qkv(2, 2, 300, 450, D, dt, seed=D + len(tile))
        check_full(q, k, v, causal, 0.11, dt, f"tile={tile}")


# The ping-pong kernel unrolls its tile loop and pairs wave groups slot by
# slot: cover every way the loop can end (1..5 key tiles, ragged and exact)
# and query blocks shorter than one workgroup.
@pytest.mark.parametrize("tile,D,dt", [("8x1x64x2x3", 128, "bf16"), ("8x1x64x2x3", 64, "f16"),
                                       ("8x1x128x2x3", 64, "bf16"), ("8x1x96x2x3", 128, "bf16"),
                                       ("8x1x96x2x3", 128, "f16")])
@pytest.mark.parametrize("Lk", [1, 63, 64, 65, 95, 96, 97, 128, 129, 191, 192, 193, 256, 257,
                                288, 289, 320, 449, 769, 833])
def test_pingpong_tile_counts(Lk, tile, D, dt, monkeypatch):
    monkeypatch.setenv("FA_TILE", tile)
    for Lq, causal in ((1, False), (257, False), (300, True)):
        q, k, v = inputs.make_qkv(1, 2, Lq, Lk, D, dt, seed=Lk * 7 + Lq + D)
        check_full(q, k, v, causal, 0.09, dt, f"pingpong {tile} Lk={Lk}")


# The ping-pong kernel keeps its stabiliser until a lane's partial row sum
# over a tile passes 2^15, then moves it to the row max and forms the tile's
# probabilities again.  Scores here climb across the keys so that this
# happens (a) through one key whose probability alone would overflow fp16
# and (b) through a whole tile of moderately larger scores, with quiet tiles
# between and a ragged last tile.
def _climbing_scores(Lq, Lk, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    t = torch.zeros(Lk)
    t[96:] = 40.0                 # every probability about 2^5: no rescale
    t[200] = 200.0                # one key about 2^26 above the stabiliser
    t[288:384] = 300.0            # a tile of keys about 2^13 above it
    t[384:] = 295.0
    q = 1.0 + 0.05 * torch.randn(1, 2, Lq, D, generator=g)
    k = t.view(1, 1, Lk, 1) / D + 0.02 * torch.randn(1, 2, Lk, D, generator=g)
    v = torch.randn(1, 2, Lk, D, generator=g)
    return (x.to(DT[dt]) for x in (q, k, v))


@pytest.mark.parametrize("tile,D,dt", [("8x1x96x2x3", 128, "bf16"), ("8x1x96x2x3", 128, "f16"),
                                       ("8x1x128x2x3", 64, "f16"), ("8x1x64x2x3", 128, "bf16")])
def test_pingpong_stabiliser_moves(tile, D, dt, monkeypatch):
    monkeypatch.setenv("FA_TILE", tile)
    for Lq, Lk, causal in ((300, 700, False), (700, 700, True)):
        q, k, v = _climbing_scores(Lq, Lk, D, dt, seed=D + Lq)
        check_full(q, k, v, causal, 0.09, dt, f"pingpong stabiliser {tile}")


# Full-size shapes beyond the five workloads, served by the large-grid
# kernels: D=64 over 16K keys (128-key ping-pong tiles; with the peaky keys
# the stabiliser moves many times along a row) and fp16 at D=128 (64- and
# 96-key ping-pong tiles); sampled rows against the oracle.
EXTRA_FULL = [((1, 32, 16384, 16384, 64, "bf16"), False),
              ((1, 32, 16384, 16384, 64, "f16"), True),
              ((4, 16, 4096, 4096, 128, "f16"), False),
              ((4, 16, 4096, 4096, 128, "f16"), True)]


@pytest.mark.parametrize("shape,causal", EXTRA_FULL,
                         ids=[f"{'x'.join(map(str, s))}-{'causal' if c else 'noncausal'}"
                              for s, c in EXTRA_FULL])
def test_large_grid_sampled(shape, causal):
    B, H, Lq, Lk, D, dt = shape
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + D + int(causal),
                              peaky_frac=0.01, peaky_factor=8.0)
    say(f"[parity] large grid {shape} causal={causal} kernel="
        f"{fa.fa_kernel_name(B, H, Lq, Lk, D, int(causal), scale, fa.dtype_code(q.dtype))}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    ids = inputs.sample_rows(B, H, Lq, n_random=16, seed=D, tile=128, heads=range(0, B * H, 3))
    ro, rl = oracle.attention_rows(to64(q), to64(k), to64(v), ids.numpy(), causal, scale)
    go = to64(o.reshape(-1, D)[ids])
    gl = lse.reshape(-1)[ids].double().numpy()
    eo, el = np.abs(go - ro).max(), np.abs(gl - rl).max()
    say(f"[parity]   rows={ids.numel()} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    assert eo <= TOL_O[dt], eo
    assert el <= TOL_LSE, el


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5, 1e-3])
def test_scale_values(scale):
    q, k, v = inputs.make_qkv(1, 2, 150, 200, 64, "bf16", seed=11)
    for causal in (False, True):
        check_full(q, k, v, causal, scale, "bf16", f"scale={scale}")


# Very large scales: scores span hundreds of binary orders, so the ping-pong
# kernel's stabiliser moves on many tiles and most probabilities underflow.
@pytest.mark.parametrize("scale", [4.0, 20.0])
@pytest.mark.parametrize("tile,D,dt", [("8x1x96x2x3", 128, "bf16"), ("8x1x64x2x3", 128, "f16"),
                                       ("8x1x128x2x3", 64, "bf16"), (None, 64, "f16")])
def test_large_scales(scale, tile, D, dt, monkeypatch):
    if tile is not None:
        monkeypatch.setenv("FA_TILE", tile)
    q, k, v = inputs.make_qkv(1, 2, 300, 700, D, dt, seed=int(scale) + D)
    for causal in (False, True):
        check_full(q, k, v, causal, scale, dt, f"scale={scale} tile={tile}")


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("Lk", [4000, 4001, 4096])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_q_zero_gives_log_lk(Lk, dt):
    """Q = 0: every score is 0, so LSE = ln Lk and O is the mean of V
    (this catches keys past Lk leaking into the sum)."""
    say(f"[closed] Q=0 Lk={Lk} {dt}")
    _, k, v = inputs.make_qkv(1, 2, 70, Lk, 64, dt, seed=Lk)
    q = torch.zeros(1, 2, 70, 64, dtype=DT[dt])
    o, lse = gpu_forward(q, k, v, False, 0.125)
    np.testing.assert_allclose(lse.double().numpy(), math.log(Lk), atol=TOL_LSE)
    mean = to64(v).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(to64(o), np.broadcast_to(mean, o.shape),
                               atol=TOL_O[dt])
    # causal: LSE_i = ln(i + 1)
    o, lse = gpu_forward(q, k, v, True, 0.125)
    want = np.log(np.arange(1, 71, dtype=np.float64))
    np.testing.assert_allclose(lse.double().numpy(),
                               np.broadcast_to(want, lse.shape), atol=TOL_LSE)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_causal_row0_is_v0_exactly(dt, D):
    say(f"[closed] causal row 0 {dt} D={D}")
    q, k, v = inputs.make_qkv(2, 3, 200, 200, D, dt, seed=5)
    o, lse = gpu_forward(q, k, v, True, 1.0 / math.sqrt(D))
    assert torch.equal(o[:, :, 0, :], v[:, :, 0, :])
    s00 = (to64(q)[:, :, 0] * to64(k)[:, :, 0]).sum(-1) / math.sqrt(D)
    np.testing.assert_allclose(lse[:, :, 0].double().numpy(), s00, atol=TOL_LSE)


def test_constant_v_rows():
    say("[closed] constant V")
    q, k, _ = inputs.make_qkv(1, 2, 300, 300, 128, "bf16", seed=6)
    row = torch.randn(1, 2, 1, 128).to(torch.bfloat16)
    v = row.expand(1, 2, 300, 128).contiguous()
    for causal in (False, True):
        o, _ = gpu_forward(q, k, v, causal, 0.088)
        np.testing.assert_allclose(to64(o), np.broadcast_to(to64(row), o.shape),
                                   atol=TOL_O["bf16"])


# ------------------------------------------------ memory safety, determinism

def test_no_writes_outside_outputs():
    """Canary bands around O and LSE stay untouched (ragged Lq tail)."""
    say("[safety] canaries")
    B, H, Lq, Lk, D = 1, 2, 197, 301, 128
    q, k, v = (t.cuda() for t in inputs.make_qkv(B, H, Lq, Lk, D, "bf16", 8))
    pad = 4096
    n_o = B * H * Lq * D
    o_buf = torch.full((n_o + 2 * pad,), float("nan"), dtype=torch.bfloat16,
                       device="cuda")
    l_buf = torch.full((B * H * Lq + 2 * pad,), -7.0, dtype=torch.float32,
                       device="cuda")
    o = o_buf[pad:pad + n_o].view(B, H, Lq, D)
    lse = l_buf[pad:pad + B * H * Lq].view(B, H, Lq)
    for causal in (False, True):
        fa.forward(q, k, v, causal=causal, scale=0.09, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isnan(o_buf[:pad]).all() and torch.isnan(o_buf[-pad:]).all()
        assert (l_buf[:pad] == -7.0).all() and (l_buf[-pad:] == -7.0).all()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_bitwise_deterministic():
    say("[safety] determinism")
    q, k, v = (t.cuda() for t in inputs.make_qkv(2, 4, 1000, 1000, 128, "bf16", 9))
    outs = []
    for _ in range(3):
        o, lse = fa.forward(q, k, v, causal=True)
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_side_stream_and_no_lse():
    say("[api] side stream, lse=NULL")
    q, k, v = inputs.make_qkv(1, 2, 256, 384, 64, "f16", 10)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.forward(dq, dk, dv, causal=False, want_lse=False)
    s.synchronize()
    assert lse is None
    ro, _ = oracle.attention(to64(q), to64(k), to64(v), False, 0.125)
    assert np.abs(to64(o.cpu()) - ro).max() <= TOL_O["f16"]


def test_host_pointer_is_rejected():
    say("[api] host pointer")
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    d = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(d)
    rc = fa.fa_fwd(q.data_ptr(), d.data_ptr(), d.data_ptr(), o.data_ptr(), None,
                   1, 1, 64, 64, 64, 0, 0.125, 2, None)
    assert rc == 8


def test_native_library_is_the_one_loaded():
    """The HIP library in the package is what runs (no fallback exists)."""
    lib = fa.load()
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(fa._lib.LIB_PATH) in maps
    hip = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hip) == 1, hip   # one HIP runtime shared with torch
    assert lib is not None


# Seeded random shapes across kernels, masks and tiles: Lq, Lk drawn from
# 1..700 (ragged against every tile size), D in {64, 128}, bf16/fp16, causal
# or not, sometimes a window, and a forced tile for the MFMA kernels (the
# ping-pong tiles only where they are built).  Every output element against
# the oracle.
def _random_cases(n=32, seed=2024):
    g = np.random.default_rng(seed)
    tiles = {64: ["8x1x128x2x3", "8x1x64x2x3", "4x1x64x2x2", "8x1x64x2x2", "4x2x64x1x2", None],
             128: ["8x1x96x2x3", "8x1x64x2x3", "4x1x64x2x2", "8x1x64x2x2", "4x2x64x1x2", None]}
    cases = []
    for i in range(n):
        D = int(g.choice([64, 128]))
        dt = str(g.choice(["bf16", "f16"]))
        Lq, Lk = int(g.integers(1, 701)), int(g.integers(1, 701))
        causal = bool(g.integers(0, 2))
        window = None
        if g.random() < 0.3:
            window = (int(g.integers(0, 300)), int(g.integers(-1, 50)))
        tile = tiles[D][int(g.integers(0, len(tiles[D])))]
        cases.append((i, 1 + int(g.integers(0, 2)), 1 + int(g.integers(0, 3)), Lq, Lk, D, dt,
                      causal, window, tile))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"r{c[0]}")
def test_random_shapes(case, monkeypatch):
    i, B, H, Lq, Lk, D, dt, causal, window, tile = case
    if tile is not None and window is None:
        monkeypatch.setenv("FA_TILE", tile)
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=1000 + i)
    say(f"[parity] random r{i}: B={B} H={H} Lq={Lq} Lk={Lk} D={D} {dt} causal={causal} "
        f"window={window} tile={tile if window is None else 'auto'}")
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o, lse = fa.forward(dq, dk, dv, causal=causal, scale=scale,
                        window=None if window is None else
                        (window[0], None if window[1] < 0 else window[1]))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to64(q), to64(k), to64(v), causal, scale, window=window)
    go, gl = to64(o.cpu()), lse.cpu().double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty)
    assert np.all(go[empty] == 0)
    eo = float(np.abs(go - ro).max())
    el = float(np.abs(gl[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    say(f"[parity]   max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O[dt], eo
    assert el <= TOL_LSE, el
