"""fa_bwd_noalloc (the allocation-free backward) against fa_bwd, through the
C ABI.  Both run the same kernels in the same order; only the home of the
per-row delta differs (a caller workspace vs the library's fixed scratch), so
the gradients must agree bit for bit.  Calls follow each other on one GPU,
the later ones smaller, so a stale scratch would show."""
import sys

import pytest
import torch

import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import inputs

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (B, H, Lq, Lk, D, dtype, causal): the first fills the scratch exactly
# (B*H*Lq = FA_NOALLOC_MAX_ROWS), the later ones are smaller
CASES = [
    (1, 512, 4096, 64, 64, "bf16", False),
    (2, 4, 1000, 700, 128, "bf16", True),
    (1, 2, 300, 333, 64, "f16", False),
    (1, 1, 77, 130, 64, "f32", True),
]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def _grads(entry, q, k, v, o, lse, g, causal, scale, stream):
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
              g.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    tail = (B, H, Lq, Lk, D, int(causal), float(scale), fa.dtype_code(q.dtype),
            stream.cuda_stream)
    if entry == "noalloc":
        rc = fa.fa_bwd_noalloc(*common, *tail)
    else:
        delta = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
        rc = fa.fa_bwd(*common, delta.data_ptr(), *tail)
    assert rc == 0, fa.fa_status_string(rc)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_matches_fa_bwd_on_consecutive_calls():
    assert CASES[0][0] * CASES[0][1] * CASES[0][2] == fa.FA_NOALLOC_MAX_ROWS
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for B, H, Lq, Lk, D, dt, causal in CASES:
        say(f"[noalloc] B={B} H={H} Lq={Lq} Lk={Lk} D={D} {dt} causal={causal}")
        scale = D ** -0.5
        q, k, v = (t.to(dev) for t in inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=Lq + Lk))
        g = inputs.make_dout(B, H, Lq, D, dt, seed=Lq).to(dev)
        o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
        ref = _grads("fa_bwd", q, k, v, o, lse, g, causal, scale, stream)
        for rep in range(2):
            got = _grads("noalloc", q, k, v, o, lse, g, causal, scale, stream)
            for name, a, b in zip(("dq", "dk", "dv"), got, ref):
                assert torch.isfinite(a.float()).all(), name
                assert torch.equal(a, b), (name, rep, (a.float() - b.float()).abs().max().item())
        say("[noalloc]   bitwise equal to fa_bwd (2 calls)")
        del q, k, v, g, o, lse, ref, got
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_call_past_its_scratch():
    dev = torch.device("cuda:0")
    B, H, Lq, Lk, D = 1, 1, fa.FA_NOALLOC_MAX_ROWS + 1, 64, 64
    t = torch.empty(16, device=dev, dtype=torch.bfloat16)
    p = t.data_ptr()
    rc = fa.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, B, H, Lq, Lk, D, 0, 0.125, 2,
                           torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 11
