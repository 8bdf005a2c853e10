"""GPU parity of the persistent ping-pong kernel (pipe 5) against the oracle.

One workgroup per CU runs query blocks g, g + G, g + 2G, ... as one stream
of key tiles, so what is specific to it is the hand-over between blocks: the
next block's Q staged through LDS, the previous block's O stored (through
LDS) at the first tile of the next one, the row state reset, loads that run
ahead into the next block, and workgroups that get different numbers of
blocks.  The shapes below have at least as many 256-row blocks as the part
has CUs (the kernel's launch condition) and cover 4 and 5 key tiles per block
(every tile then sits at a block boundary), ragged Lq and Lk, both I/O types,
peaky keys (the stabiliser moves), large scales and the stabiliser test of
the ping-pong kernel.  Whole outputs are compared.
"""
import math

import pytest
import torch

import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import inputs

from test_parity_gpu import TOL_LSE, TOL_O, check_whole, say

pytestmark = pytest.mark.gpu

PERS = "8x1x64x2x5"


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def blocks(B, H, Lq):
    return B * H * ((Lq + 255) // 256)


CASES = [
    # B, H, Lq, Lk, dtype, peaky, scale
    (2, 64, 1024, 300, "bf16", False, None),     # 5 key tiles, ragged
    (1, 75, 1000, 256, "bf16", False, None),     # 4 key tiles; 300 blocks (uneven)
    (3, 100, 700, 513, "f16", False, None),      # ragged Lq and Lk
    (1, 128, 1024, 1024, "bf16", True, None),    # peaky: the stabiliser moves
    (1, 64, 2048, 640, "bf16", False, 0.5),      # large scale
    (1, 32, 4096, 4096, "f16", True, None),      # long rows, 2 blocks per workgroup
    (8, 16, 1024, 4096, "f16", False, None),     # 32 tiles, 2 blocks per workgroup
    (2, 64, 1000, 777, "bf16", False, None),     # ragged Lq and Lk, 13 tiles
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-{c[4]}" for c in CASES])
def test_persistent_whole_output(case, monkeypatch):
    B, H, Lq, Lk, dt, peaky, sc = case
    if blocks(B, H, Lq) < cus():
        pytest.skip("fewer query blocks than CUs")
    monkeypatch.setenv("FA_TILE", PERS)
    D = 128
    scale = sc or 1.0 / math.sqrt(D)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + Lk + H,
                              peaky_frac=0.01 if peaky else 0.0, peaky_factor=8.0)
    eo, el, over = check_whole(q, k, v, False, scale, dt, f"persistent {case}", heads_per_chunk=32)
    assert "ppp8w" in fa.fa_kernel_name(B, H, Lq, Lk, D, 0, scale, fa.dtype_code(q.dtype))
    assert eo <= TOL_O[dt] and over == 0, (eo, over)
    assert el <= TOL_LSE, el


def test_persistent_stabiliser_moves(monkeypatch):
    """Scores that climb along the keys (one key 2^26 above the stabiliser,
    then a whole tile 2^13 above it) in every head: the row state must reset
    cleanly at each block boundary."""
    monkeypatch.setenv("FA_TILE", PERS)
    B, H, Lq, Lk, D = 1, 2 * cus(), 300, 700, 128
    g = torch.Generator().manual_seed(5)
    t = torch.zeros(Lk)
    t[96:] = 40.0
    t[200] = 200.0
    t[288:384] = 300.0
    t[384:] = 295.0
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        q = (1.0 + 0.05 * torch.randn(B, H, Lq, D, generator=g)).to(tdt)
        k = (t.view(1, 1, Lk, 1) / D + 0.02 * torch.randn(B, H, Lk, D, generator=g)).to(tdt)
        v = torch.randn(B, H, Lk, D, generator=g).to(tdt)
        eo, el, over = check_whole(q, k, v, False, 0.09, dt, "persistent stabiliser",
                                   heads_per_chunk=64)
        assert eo <= TOL_O[dt] and over == 0, (eo, over)
        assert el <= TOL_LSE, el


def test_persistent_is_the_default_for_short_rows():
    """D=128 non-causal rows of 193..2048 keys with two or more blocks per
    workgroup take the persistent kernel; longer rows, causal calls and a
    single block per workgroup keep the ping-pong kernel."""
    n = cus()
    H = 2 * n // 4          # B=1, Lq=1024: 4 blocks per head -> 2 blocks per CU
    assert "ppp8w" in fa.fa_kernel_name(1, H, 1024, 1024, 128, 0, 0.088, 2)
    assert "ppp8w" in fa.fa_kernel_name(1, H, 1024, 193, 128, 0, 0.088, 1)
    assert "ppp8w" in fa.fa_kernel_name(1, H, 1024, 2048, 128, 0, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H, 1024, 2049, 128, 0, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H, 1024, 4096, 128, 0, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H, 1024, 1024, 128, 1, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H, 1024, 192, 128, 0, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H // 2, 1024, 1024, 128, 0, 0.088, 2)
    assert "ppp8w" not in fa.fa_kernel_name(1, H, 1024, 1024, 64, 0, 0.088, 2)


def test_persistent_default_path_and_canaries():
    """The default choice on a short-row shape, whole output, with canary
    bands around O and LSE (ragged last block: Lq = 1000)."""
    n = cus()
    B, H, Lq, Lk, D = 1, n // 2, 1000, 777, 128
    assert "ppp8w" in fa.fa_kernel_name(B, H, Lq, Lk, D, 0, 0.09, 2)
    q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, "bf16", seed=77)
    eo, el, over = check_whole(q, k, v, False, 0.09, "bf16", "persistent default", heads_per_chunk=32)
    assert eo <= TOL_O["bf16"] and over == 0, (eo, over)
    assert el <= TOL_LSE, el
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    pad = 8192
    n_o = B * H * Lq * D
    o_buf = torch.full((n_o + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((B * H * Lq + 2 * pad,), -7.0, dtype=torch.float32, device="cuda")
    o = o_buf[pad:pad + n_o].view(B, H, Lq, D)
    lse = l_buf[pad:pad + B * H * Lq].view(B, H, Lq)
    fa.forward(dq, dk, dv, causal=False, scale=0.09, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(o_buf[:pad]).all() and torch.isnan(o_buf[-pad:]).all()
    assert (l_buf[:pad] == -7.0).all() and (l_buf[-pad:] == -7.0).all()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_persistent_bitwise_deterministic(monkeypatch):
    monkeypatch.setenv("FA_TILE", PERS)
    q, k, v = (t.cuda() for t in inputs.make_qkv(1, cus(), 1024, 900, 128, "bf16", 19))
    outs = []
    for _ in range(3):
        o, lse = fa.forward(q, k, v, causal=False)
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_persistent_refuses_what_it_is_not_built_for(monkeypatch):
    """Forced onto a call it does not cover (fewer blocks than CUs, causal,
    D=64, under 4 key tiles), the kernel is not launched: the call reports a
    launch error and writes nothing."""
    monkeypatch.setenv("FA_TILE", PERS)
    for B, H, Lq, Lk, D, causal in ((1, 2, 256, 512, 128, False),
                                    (1, cus(), 1024, 512, 128, True),
                                    (1, cus(), 1024, 512, 64, False),
                                    (1, cus(), 1024, 192, 128, False)):
        q, k, v = (t.cuda() for t in inputs.make_qkv(B, H, Lq, Lk, D, "bf16", 3))
        o = torch.full_like(q, 7.0)
        say(f"[persistent] refused: {(B, H, Lq, Lk, D, causal)}")
        with pytest.raises(RuntimeError):
            fa.forward(q, k, v, causal=causal, out=o)
        torch.cuda.synchronize()
        assert (o == 7.0).all()
