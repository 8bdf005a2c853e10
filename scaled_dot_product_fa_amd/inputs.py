"""Seeded synthetic inputs for the attention forward, shared by tests and bench.

This module only draws numbers and names workloads; it performs none of the
attention arithmetic, so both the GPU path and the CPU reference can consume
its tensors without sharing any method code.

Recipe (all on the CPU, ``torch.Generator('cpu').manual_seed(seed)``):
  * draw Q, then K, then V with ``torch.randn(shape, float32)`` -- iid N(0, 1);
  * for the long-context stress workload, per (b, h) pick ``round(frac * Lk)``
    key rows with a seeded ``randperm`` and multiply them by ``factor`` in
    float32 (x8 is exact in bf16/fp16), which makes the softmax peaky;
  * cast to the I/O dtype with round-to-nearest-even (torch's ``.to``).
A key-trimmed variant (Lk not a multiple of the tile size) takes the first
``Lk`` keys of a longer draw and makes them contiguous.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention shape with its I/O dtype, scale, seed and input structure."""
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    D: int
    dtype: str
    scale: float
    seed: int
    modes: tuple          # subset of ("noncausal", "causal")
    peaky_frac: float = 0.0
    peaky_factor: float = 1.0
    draw_Lk: int = 0      # >Lk: keys drawn at this length, first Lk kept

    def flops(self, causal: bool) -> float:
        """4*B*H*Lq*Lk*D (two GEMMs, forward only), halved when causal."""
        f = 4.0 * self.B * self.H * self.Lq * self.Lk * self.D
        return f / 2.0 if causal else f

    def io_bytes(self) -> int:
        """Read Q, K, V once and write O and the fp32 LSE once."""
        elem = torch.tensor([], dtype=DTYPES[self.dtype]).element_size()
        return (elem * self.B * self.H * (2 * self.Lq + 2 * self.Lk) * self.D
                + 4 * self.B * self.H * self.Lq)


# The five workloads: a tiny fp32 case, a small LLM head, the mid training
# shape, the 16K long-context stress case and an fp16 cross-attention case
# (also with a ragged key length of 4000).
CONFIGS = {
    "tiny": Workload("tiny", 1, 2, 128, 128, 64, "f32", 1.0 / math.sqrt(64), 1,
                     ("noncausal", "causal")),
    "small": Workload("small", 2, 8, 1024, 1024, 64, "bf16", 1.0 / 8, 2,
                      ("noncausal", "causal")),
    "mid": Workload("mid", 4, 16, 4096, 4096, 128, "bf16",
                    1.0 / math.sqrt(128), 3, ("noncausal", "causal")),
    "long": Workload("long", 1, 32, 16384, 16384, 128, "bf16",
                     1.0 / math.sqrt(128), 4, ("causal", "noncausal"),
                     peaky_frac=0.01, peaky_factor=8.0),
    "xattn": Workload("xattn", 8, 16, 1024, 4096, 64, "f16", 1.0 / 8, 5,
                      ("noncausal",)),
    "xattn_lk4000": Workload("xattn_lk4000", 8, 16, 1024, 4000, 64, "f16",
                             1.0 / 8, 5, ("noncausal",), draw_Lk=4096),
}


def make_qkv(B: int, H: int, Lq: int, Lk: int, D: int, dtype: str = "bf16",
             seed: int = 0, peaky_frac: float = 0.0,
             peaky_factor: float = 1.0, draw_Lk: int = 0):
    """Seeded CPU tensors q [B,H,Lq,D], k and v [B,H,Lk,D] in ``dtype``."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    Lk_draw = max(draw_Lk, Lk)
    q = torch.randn((B, H, Lq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Lk_draw, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Lk_draw, D), generator=g, dtype=torch.float32)
    if peaky_frac > 0.0:
        n_big = int(round(peaky_frac * Lk_draw))
        for b in range(B):
            for h in range(H):
                idx = torch.randperm(Lk_draw, generator=g)[:n_big]
                k[b, h, idx, :] *= peaky_factor
    if Lk_draw != Lk:
        k = k[:, :, :Lk, :].contiguous()
        v = v[:, :, :Lk, :].contiguous()
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def make_dout(B: int, H: int, Lq: int, D: int, dtype: str = "bf16",
              seed: int = 0):
    """Seeded incoming gradient dO [B,H,Lq,D] (iid N(0, 1), cast RNE), from
    its own generator so that q, k, v are the same draws as make_qkv's."""
    g = torch.Generator("cpu").manual_seed(int(seed) * 2654435761 % (1 << 63) + 17)
    return torch.randn((B, H, Lq, D), generator=g,
                       dtype=torch.float32).to(DTYPES[dtype])


def workload_inputs(w: Workload):
    """The seeded inputs of a named workload (CPU tensors)."""
    return make_qkv(w.B, w.H, w.Lq, w.Lk, w.D, w.dtype, w.seed, w.peaky_frac,
                    w.peaky_factor, w.draw_Lk)


def sample_rows(B: int, H: int, Lq: int, n_random: int = 64, seed: int = 0,
                tile: int = 64, heads=None):
    """Flat row ids (b*H + h)*Lq + i for sampled-row checks at full size.

    Per selected head: rows 0 and 1, the first and last row of every
    ``tile``-row block boundary near the start, the middle and the end, the
    last row, plus ``n_random`` seeded rows.  Heads default to all of them.
    """
    g = torch.Generator("cpu").manual_seed(int(seed) + 7919)
    fixed = {0, 1, Lq - 1, Lq - 2, Lq // 2}
    for t in (1, 2, 3, Lq // tile // 2, Lq // tile - 1):
        for i in (t * tile - 1, t * tile):
            if 0 <= i < Lq:
                fixed.add(i)
    fixed = sorted(i for i in fixed if 0 <= i < Lq)
    if heads is None:
        heads = range(B * H)
    ids = []
    for bh in heads:
        rnd = torch.randint(0, Lq, (n_random,), generator=g).tolist()
        for i in sorted(set(fixed) | set(rnd)):
            ids.append(bh * Lq + i)
    return torch.tensor(ids, dtype=torch.int64)


def sha256_of(*tensors) -> str:
    """Hex digest of the raw bytes of the given CPU tensors, in order."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
