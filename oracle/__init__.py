"""CPU fp64 reference for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path
(``scaled_dot_product_fa_amd``) never imports it and shares no code with it.

The arithmetic lives in ``fa_oracle.c`` (plain C, IEEE double, OpenMP over
rows).  This module builds that file with gcc and marshals numpy arrays to
it; it does no attention arithmetic of its own.

Definition followed: the three phases of "Triton Ascend Attention", section
"standard attention computation flow" (scores Q K^T scaled, softmax with rows
summing to one, weighted sum with V), plus the natural-log row statistic
m + log(l) that the FlashAttention-2 forward article's kernel epilogue stores.
Causal masking keeps key j for query i when j <= i ("flash-attention-kernel"
skill page, pitfalls; the article's _attn_fwd_inner mask).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_F64P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)
_I64 = ctypes.c_int64


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into ``out``."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    lib.oracle_attention.argtypes = [_F64P, _F64P, _F64P, _F64P, _F64P,
                                     _I64, _I64, _I64, _I64, _I64,
                                     ctypes.c_int, ctypes.c_double]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [_F64P, _F64P, _F64P, _I64P, _I64,
                                          _F64P, _F64P, _I64, _I64, _I64,
                                          _I64, _I64, ctypes.c_int,
                                          ctypes.c_double]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_win.argtypes = [_F64P, _F64P, _F64P, _F64P, _F64P,
                                         _I64, _I64, _I64, _I64, _I64,
                                         ctypes.c_int, _I64, _I64,
                                         ctypes.c_double]
    lib.oracle_attention_win.restype = ctypes.c_int
    lib.oracle_attention_rows_win.argtypes = [_F64P, _F64P, _F64P, _I64P, _I64,
                                              _F64P, _F64P, _I64, _I64, _I64,
                                              _I64, _I64, ctypes.c_int, _I64,
                                              _I64, ctypes.c_double]
    lib.oracle_attention_rows_win.restype = ctypes.c_int
    lib.oracle_probs.argtypes = [_F64P, _F64P, _F64P, _I64, _I64, _I64, _I64,
                                 _I64, ctypes.c_int, ctypes.c_double]
    lib.oracle_probs.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [_F64P] * 8 + [_I64] * 5 + [
        ctypes.c_int, ctypes.c_double]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention_bwd_win.argtypes = [_F64P] * 8 + [_I64] * 5 + [
        ctypes.c_int, _I64, _I64, ctypes.c_double]
    lib.oracle_attention_bwd_win.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the compiled oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_F64P)


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, H, Lq, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    return B, H, Lq, k.shape[2], D


def attention(q, k, v, causal: bool = False, scale: float | None = None,
              lib=None, window=None):
    """Full fp64 forward.  Returns (o [B,H,Lq,D], lse [B,H,Lq]).

    ``window=(wl, wr)`` keeps key j for query i only when i - wl <= j <= i + wr
    (a negative bound is no bound)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Lq, Lk, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty((B, H, Lq, D), dtype=np.float64)
    lse = np.empty((B, H, Lq), dtype=np.float64)
    lib = lib or load()
    if window is None:
        rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(lse), B, H, Lq, Lk, D,
                                  int(bool(causal)), float(scale))
    else:
        rc = lib.oracle_attention_win(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(lse), B, H, Lq, Lk, D,
                                      int(bool(causal)), int(window[0]),
                                      int(window[1]), float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return o, lse


def attention_rows(q, k, v, row_ids, causal: bool = False,
                   scale: float | None = None, lib=None, window=None):
    """Selected rows.  row_ids are flat (b*H + h)*Lq + i indices.

    Returns (o_rows [n, D], lse_rows [n]); each row equals the matching row of
    :func:`attention` (same ``window`` convention).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Lq, Lk, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64))
    n = ids.size
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    rc = (lib or load()).oracle_attention_rows_win(
        _ptr(q), _ptr(k), _ptr(v), ids.ctypes.data_as(_I64P), n, _ptr(o),
        _ptr(lse), B, H, Lq, Lk, D, int(bool(causal)), wl, wr, float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed ({rc})")
    return o, lse


def probs(q, k, causal: bool = False, scale: float | None = None, lib=None):
    """The probability matrix P [B,H,Lq,Lk] (zero where masked)."""
    q, k = _f64(q), _f64(k)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    p = np.empty((B, H, Lq, Lk), dtype=np.float64)
    rc = (lib or load()).oracle_probs(_ptr(q), _ptr(k), _ptr(p), B, H, Lq, Lk,
                                      D, int(bool(causal)), float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_probs failed ({rc})")
    return p


def attention_bwd(q, k, v, dout, causal: bool = False,
                  scale: float | None = None, lib=None, with_delta=False,
                  window=None):
    """fp64 gradients (dq, dk, dv) of the forward for an incoming gradient
    ``dout`` of o (lse takes no gradient).  The plain chain rule through the
    forward definition; the C source states each step.  With ``with_delta``
    also returns delta [B,H,Lq], delta_i = sum_j p_ij (dout_i . v_j).
    ``window=(wl, wr)`` as for :func:`attention`."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Lq, Lk, D = _shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    delta = np.empty((B, H, Lq), dtype=np.float64)
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    rc = (lib or load()).oracle_attention_bwd_win(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(delta), B, H, Lq, Lk, D, int(bool(causal)), wl, wr, float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
    if with_delta:
        return dq, dk, dv, delta
    return dq, dk, dv


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all cores)."""
    return int((lib or load()).oracle_num_threads())
