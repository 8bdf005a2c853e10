"""Tensors past 2^31 elements (byte offsets past 4 GiB): B*H = 65536 heads of
256 x 128 bf16, 4 GiB per tensor.  The forward and the backward run once at
full size; heads at the start, middle and end are compared with the oracle,
which catches any 32-bit index that wraps.  Inputs are drawn on the device
from a seeded generator (iid N(0, 1), cast to bf16)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_fa_amd as fa

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def test_more_than_2_pow_31_elements():
    dev = torch.device("cuda:0")
    B, H, L, D = 256, 256, 256, 128
    assert B * H * L * D == 1 << 31
    scale = 1.0 / math.sqrt(D)
    gen = torch.Generator(device=dev).manual_seed(2024)

    def draw():
        return torch.randn((B, H, L, D), generator=gen, device=dev,
                           dtype=torch.float32).to(torch.bfloat16)

    q, k, v, g = draw(), draw(), draw(), draw()
    say(f"[large] B={B} H={H} L={L} D={D} bf16 causal, {q.numel()} elements per tensor")
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, g, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B // 2, 17), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        f64 = lambda t: t[sl].cpu().double().numpy()
        ro, rl = oracle.attention(f64(q), f64(k), f64(v), True, scale)
        eo = float(np.abs(f64(o) - ro).max())
        el = float(np.abs(lse[sl].cpu().double().numpy() - rl).max())
        rq, rk, rv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(g), True, scale)
        errs = [float(np.abs(f64(a) - r).max() / np.abs(r).max())
                for a, r in ((dq, rq), (dk, rk), (dv, rv))]
        say(f"[large]   head ({b},{h}) max|dO|={eo:.2e} max|dLSE|={el:.2e} "
            f"grads/max|ref|={errs[0]:.2e} {errs[1]:.2e} {errs[2]:.2e}")
        assert eo <= 2e-2 and el <= 1e-3
        assert max(errs) <= 2e-2
