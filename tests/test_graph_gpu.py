"""The forward and backward under HIP graph capture: captured once, replayed
several times with eager work and synchronisations in between, every replay
equal bit for bit to the eager result (the library enqueues only kernels: no
allocations, memsets or host synchronisation inside a call)."""
import math

import pytest
import torch

import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,dt,causal", [(128, "bf16", True), (64, "f16", False)])
def test_forward_backward_graph_replay(D, dt, causal):
    dev = torch.device("cuda:0")
    B, H, Lq, Lk = 2, 4, 640, 700
    scale = 1.0 / math.sqrt(D)
    q, k, v = (t.to(dev) for t in inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=D + Lq))
    g = inputs.make_dout(B, H, Lq, D, dt, seed=D).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def call():
        fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        fa.backward(q, k, v, o, lse, g, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,
                    delta=delta)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), (rep, name)
