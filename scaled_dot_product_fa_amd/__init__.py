"""MI355X (gfx950) FlashAttention-2 forward, and its backward.

``forward(q, k, v, causal=False, scale=None)`` returns ``(o, lse)`` for
contiguous ``[B, H, L, D]`` device tensors (bf16, fp16 or fp32; D = 64 or
128); ``backward(q, k, v, o, lse, dout, ...)`` returns ``(dq, dk, dv)``.  PyTorch provides the device memory and the stream; the computation is
the HIP kernels in ``libfa.so`` behind the C ABI of ``include/fa.h``.
"""
from __future__ import annotations

import math

from ._lib import (FA_BF16, FA_F16, FA_F32, FA_NOALLOC_MAX_ROWS, FaError,
                   fa_bwd, fa_bwd_ex, fa_bwd_kernel_name, fa_bwd_noalloc, fa_fwd,
                   fa_fwd_ex, fa_kernel_name, fa_status_string, fa_version, load)

__all__ = ["forward", "backward", "fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_ex",
           "fa_bwd_noalloc", "FA_NOALLOC_MAX_ROWS",
           "fa_kernel_name",
           "fa_bwd_kernel_name", "fa_status_string", "fa_version", "FaError",
           "dtype_code", "load"]


def dtype_code(dtype) -> int:
    """enum fa_dtype value of a torch dtype."""
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16,
             torch.bfloat16: FA_BF16}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[dtype]


def forward(q, k, v, causal: bool = False, scale: float | None = None,
            out=None, lse=None, want_lse: bool = True, stream=None,
            window=None):
    """Attention forward on the current (or given) stream.

    q [B,H,Lq,D], k/v [B,H,Lk,D] CUDA (HIP) tensors of one dtype.  Views
    with any (batch, head, row) strides work as long as D is contiguous (for
    example a [B,L,H,D] tensor transposed to [B,H,L,D]); they, and a local
    ``window=(left, right)`` (query i keeps keys i-left .. i+right; None or
    a negative bound: no bound), go through ``fa_fwd_ex``, everything else
    through ``fa_fwd``.  ``scale`` defaults to 1/sqrt(D).  Returns (o, lse)
    with o laid out like q (``empty_like``) and lse fp32 [B,H,Lq] (None when
    ``want_lse`` is False).  ``out``/``lse`` may be preallocated.  Raises
    FaError on a status other than FA_OK.
    """
    import torch
    load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D]")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
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
    if out.stride(3) != 1 or tuple(out.shape) != (B, H, Lq, D):
        raise ValueError("out must be [B, H, Lq, D] with a contiguous last dimension")
    wl, wr = (-1, -1) if window is None else (
        -1 if window[0] is None else int(window[0]),
        -1 if window[1] is None else int(window[1]))
    general = (not all(t.is_contiguous() for t in (q, k, v, out))) or wl >= 0 or wr >= 0
    lse_ptr = lse.data_ptr() if lse is not None else None
    if general:
        strides = [x for t in (q, k, v, out) for x in t.stride()[:3]]
        rc = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse_ptr, B, H, Lq, Lk, D, strides, int(bool(causal)), wl, wr,
                       float(scale), dtype_code(q.dtype), stream.cuda_stream)
    else:
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                    lse_ptr, B, H, Lq, Lk, D, int(bool(causal)), float(scale),
                    dtype_code(q.dtype), stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False,
             scale: float | None = None, dq=None, dk=None, dv=None,
             delta=None, stream=None, window=None):
    """Gradients (dq, dk, dv) of the forward for an incoming ``dout``.

    q, k, v, causal, scale and window as given to :func:`forward`; o and lse
    are what it returned; dout is like o.  Strided views (last dimension
    contiguous) and a window go through ``fa_bwd_ex``, the rest through
    ``fa_bwd``.  ``dq``/``dk``/``dv`` (laid out like q/k/v by default) and
    the fp32 [B,H,Lq] workspace ``delta`` may be preallocated.  Raises
    FaError on a status other than FA_OK.
    """
    import torch
    load()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D]")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o, dout must share one dtype")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if (tuple(k.shape) != (B, H, Lk, D) or tuple(v.shape) != (B, H, Lk, D)
            or tuple(o.shape) != (B, H, Lq, D)
            or tuple(dout.shape) != (B, H, Lq, D)):
        raise ValueError("shapes must be q/o/dout [B,H,Lq,D], k/v [B,H,Lk,D]")
    if (lse is None or not lse.is_cuda or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, Lq) or not lse.is_contiguous()):
        raise ValueError("lse must be the forward's fp32 [B, H, Lq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    wl, wr = (-1, -1) if window is None else (
        -1 if window[0] is None else int(window[0]),
        -1 if window[1] is None else int(window[1]))
    tensors = (q, k, v, o, dout, dq, dk, dv)
    general = (not all(t.is_contiguous() for t in tensors)) or wl >= 0 or wr >= 0
    if general:
        strides = [x for t in tensors for x in t.stride()[:3]]
        rc = fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                       dv.data_ptr(), delta.data_ptr(), B, H, Lq, Lk, D, strides,
                       int(bool(causal)), wl, wr, float(scale), dtype_code(q.dtype),
                       stream.cuda_stream)
    else:
        rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                    lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                    dv.data_ptr(), delta.data_ptr(), B, H, Lq, Lk, D,
                    int(bool(causal)), float(scale), dtype_code(q.dtype),
                    stream.cuda_stream)
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))
    return dq, dk, dv
