"""MI355X (gfx950) FlashAttention-2 forward.

``forward(q, k, v, causal=False, scale=None)`` returns ``(o, lse)`` for
contiguous ``[B, H, L, D]`` device tensors (bf16, fp16 or fp32; D = 64 or
128).  PyTorch provides the device memory and the stream; the computation is
the HIP kernels in ``libfa.so`` behind the C ABI of ``include/fa.h``.
"""
from __future__ import annotations

import math

from ._lib import (FA_BF16, FA_F16, FA_F32, FaError, fa_fwd, fa_kernel_name,
                   fa_status_string, fa_version, load)

__all__ = ["forward", "fa_fwd", "fa_kernel_name", "fa_status_string",
           "fa_version", "FaError", "dtype_code", "load"]


def dtype_code(dtype) -> int:
    """enum fa_dtype value of a torch dtype."""
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16,
             torch.bfloat16: FA_BF16}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[dtype]


def forward(q, k, v, causal: bool = False, scale: float | None = None,
            out=None, lse=None, want_lse: bool = True, stream=None):
    """Attention forward on the current (or given) stream.

    q [B,H,Lq,D], k/v [B,H,Lk,D] CUDA (HIP) tensors of one dtype, contiguous.
    ``scale`` defaults to 1/sqrt(D).  Returns (o, lse) with o like q and lse
    fp32 [B,H,Lq] (None when ``want_lse`` is False).  ``out``/``lse`` may be
    preallocated.  Raises FaError on a status other than FA_OK.
    """
    import torch
    load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, D) or tuple(v.shape) != (B, H, Lk, D):
        raise ValueError("k and v must be [B, H, Lk, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                lse.data_ptr() if lse is not None else None, B, H, Lq, Lk, D,
                int(bool(causal)), float(scale), dtype_code(q.dtype),
                stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))
    return out, lse
