"""ctypes binding of libfa.so: argument marshalling only.

The names match the C ABI in include/fa.h (``fa_fwd``, ``fa_fwd_ex``, ``fa_bwd``,
``fa_bwd_ex``, ``fa_bwd_noalloc``,
``fa_status_string``, ``fa_kernel_name``, ``fa_bwd_kernel_name``,
``fa_version``).  Every step of the attention forward and backward runs in
the HIP kernels; there is no Python or CPU fallback, and loading
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM",
    4: "FA_ERR_DTYPE", 5: "FA_ERR_SCALE", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ALIAS",
    8: "FA_ERR_POINTER", 9: "FA_ERR_LAUNCH", 10: "FA_ERR_STRIDE",
    11: "FA_ERR_SCRATCH",
}
FA_NOALLOC_MAX_ROWS = 1 << 21

_lib = None


class FaError(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m scaled_dot_product_fa_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                           ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                              ctypes.POINTER(ctypes.c_int64), ctypes.c_int, i64,
                              i64, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_fwd_ex.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp] * 10 + [i64] * 5 + [
        ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_ex.argtypes = [vp] * 10 + [i64] * 5 + [
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int, i64, i64, ctypes.c_float,
        ctypes.c_int, vp]
    lib.fa_bwd_ex.restype = ctypes.c_int
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i64] * 5 + [
        ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_bwd_noalloc.restype = ctypes.c_int
    lib.fa_bwd_kernel_name.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int]
    lib.fa_bwd_kernel_name.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_kernel_name.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_int]
    lib.fa_kernel_name.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def fa_fwd(q: int, k: int, v: int, o: int, lse: int | None, B: int, H: int,
           Lq: int, Lk: int, D: int, causal: int, scale: float, dtype: int,
           stream: int | None) -> int:
    """Raw call: integer device addresses in, status code out."""
    return load().fa_fwd(q, k, v, o, lse, B, H, Lq, Lk, D, int(causal),
                         float(scale), int(dtype), stream)


def fa_fwd_ex(q: int, k: int, v: int, o: int, lse: int | None, B: int, H: int,
              Lq: int, Lk: int, D: int, strides, causal: int,
              window_left: int, window_right: int, scale: float, dtype: int,
              stream: int | None) -> int:
    """Raw call: device addresses, 12 element strides (q, k, v, o; each
    batch, head, row), window bounds (-1: none); status code out."""
    arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides]) if strides is not None else None
    return load().fa_fwd_ex(q, k, v, o, lse, B, H, Lq, Lk, D, arr, int(causal),
                            int(window_left), int(window_right), float(scale),
                            int(dtype), stream)


def fa_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int,
           dk: int, dv: int, delta: int, B: int, H: int, Lq: int, Lk: int,
           D: int, causal: int, scale: float, dtype: int,
           stream: int | None) -> int:
    """Raw call: integer device addresses in, status code out."""
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Lq,
                         Lk, D, int(causal), float(scale), int(dtype), stream)


def fa_bwd_ex(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int,
              dk: int, dv: int, delta: int, B: int, H: int, Lq: int, Lk: int,
              D: int, strides, causal: int, window_left: int,
              window_right: int, scale: float, dtype: int,
              stream: int | None) -> int:
    """Raw call: device addresses, 24 element strides (q, k, v, o, dout, dq,
    dk, dv; each batch, head, row), window bounds (-1: none)."""
    arr = (ctypes.c_int64 * 24)(*[int(x) for x in strides]) if strides is not None else None
    return load().fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Lq,
                            Lk, D, arr, int(causal), int(window_left),
                            int(window_right), float(scale), int(dtype), stream)


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, lse: int, dout: int,
                   dq: int, dk: int, dv: int, B: int, H: int, Lq: int, Lk: int,
                   D: int, causal: int, scale: float, dtype: int,
                   stream: int | None) -> int:
    """Raw call of fa_bwd without a delta workspace (the library's fixed
    scratch holds it; B*H*Lq <= FA_NOALLOC_MAX_ROWS)."""
    return load().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq,
                                 Lk, D, int(causal), float(scale), int(dtype),
                                 stream)


def fa_bwd_kernel_name(B: int, H: int, Lq: int, Lk: int, D: int, causal: int,
                       scale: float, dtype: int) -> str | None:
    r = load().fa_bwd_kernel_name(B, H, Lq, Lk, D, int(causal), float(scale),
                                  int(dtype))
    return None if r is None else r.decode()


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_kernel_name(B: int, H: int, Lq: int, Lk: int, D: int, causal: int,
                   scale: float, dtype: int) -> str | None:
    r = load().fa_kernel_name(B, H, Lq, Lk, D, int(causal), float(scale),
                              int(dtype))
    return None if r is None else r.decode()


def fa_version() -> int:
    return int(load().fa_version())
