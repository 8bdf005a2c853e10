"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/fa.h declares, and rejects bad arguments on the host before any
launch (fake addresses are never dereferenced because validation fails
first)."""
import ctypes
import math
import os
import re

import pytest

import scaled_dot_product_fa_amd as fa
from scaled_dot_product_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_bwd", "fa_bwd_ex", "fa_bwd_kernel_name",
                                    "fa_bwd_noalloc",
                                    "fa_fwd", "fa_fwd_ex", "fa_kernel_name",
                                    "fa_status_string", "fa_version"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(0, 12):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"
    assert fa.fa_status_string(-1) == "unknown status"


def test_enum_values_match_header():
    text = open(HEADER).read()
    for name, val in (("FA_F32", 0), ("FA_F16", 1), ("FA_BF16", 2)):
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text)
    for code, name in _lib.STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name


# Fake, well-separated, 16-byte aligned addresses: validation must reject
# the call before anything could touch them.
Q, K, V, O, L = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40
GOOD = dict(B=1, H=2, Lq=128, Lk=128, D=64, causal=0, scale=0.125, dtype=2)


def call(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(q, k, v, o, lse, a["B"], a["H"], a["Lq"], a["Lk"],
                     a["D"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_null_pointer(which):
    assert call(**{which: None}) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(H=0), 2), (dict(Lq=0), 2), (dict(Lk=0), 2),
    (dict(B=-3), 2), (dict(Lq=(1 << 24) + 1), 2), (dict(Lk=(1 << 24) + 1), 2),
    (dict(B=1 << 13, H=1 << 12), 2),
    (dict(D=32), 3), (dict(D=96), 3), (dict(D=256), 3), (dict(D=0), 3),
    (dict(dtype=3), 4), (dict(dtype=-1), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5),
    (dict(scale=-float("inf")), 5),
])
def test_bad_arguments(kw, code):
    assert call(**kw) == code


def test_misaligned_pointers():
    assert call(q=Q + 8) == 6
    assert call(o=O + 2) == 6
    assert call(lse=L + 2) == 6


def test_aliasing_rejected():
    nbytes = 1 * 2 * 128 * 64 * 2
    assert call(o=Q) == 7                      # o on top of q
    assert call(o=K + nbytes - 16) == 7        # o overlapping the tail of k
    assert call(lse=O + 64) == 7               # lse inside o
    assert call(lse=V) == 7


def test_non_device_pointers_rejected_without_gpu():
    # plain host addresses are not device memory (and there is no GPU here)
    buf = [ctypes.create_string_buffer(1 << 16) for _ in range(5)]
    addr = [((ctypes.addressof(b) + 15) // 16) * 16 for b in buf]
    assert call(q=addr[0], k=addr[1], v=addr[2], o=addr[3], lse=addr[4]) == 8


def test_kernel_selection():
    # bf16/fp16 with a positive scale run on MFMA, everything else on VALU
    # (labels name the kernel family and its tile: pp = ping-pong, pipe =
    # software-pipelined; waves per workgroup; keys per tile)
    assert fa.fa_kernel_name(4, 16, 4096, 4096, 128, 0, 0.088, 2) == \
        "fa_fwd_mfma_bf16_d128_pp8w_bn64"
    assert fa.fa_kernel_name(1, 32, 16384, 16384, 128, 1, 0.088, 2) == \
        "fa_fwd_mfma_bf16_d128_causal_pp8w_bn96"
    assert fa.fa_kernel_name(8, 16, 1024, 4000, 64, 0, 0.125, 1) == \
        "fa_fwd_mfma_f16_d64_pp8w_bn128"
    assert fa.fa_kernel_name(2, 8, 1024, 1024, 64, 1, 0.125, 2) == \
        "fa_fwd_mfma_bf16_d64_causal_pipe4w_bn64"
    assert fa.fa_kernel_name(1, 2, 128, 128, 64, 1, 0.125, 0) == \
        "fa_fwd_valu_f32_d64_causal"
    assert fa.fa_kernel_name(1, 2, 128, 128, 64, 0, 0.0, 2) == \
        "fa_fwd_valu_bf16_d64"
    assert fa.fa_kernel_name(1, 2, 128, 128, 128, 0, -1.0, 1) == \
        "fa_fwd_valu_f16_d128"
    assert fa.fa_kernel_name(1, 2, 128, 128, 65, 0, 1.0, 2) is None
    assert fa.fa_kernel_name(1, 2, 128, 128, 64, 0, math.nan, 2) is None
    assert fa.fa_kernel_name(1, 2, 0, 128, 64, 0, 1.0, 2) is None


def test_forward_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_version():
    assert fa.fa_version() >= 200


# ---- fa_bwd: the same host-side validation --------------------------------

DO, DQ, DK, DV, DL = 6 << 40, 7 << 40, 8 << 40, 9 << 40, 10 << 40


def bcall(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL,
          **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, a["B"], a["H"],
                     a["Lq"], a["Lk"], a["D"], a["causal"], a["scale"],
                     a["dtype"], None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "dout", "dq",
                                   "dk", "dv", "delta"])
def test_bwd_null_pointer(which):
    assert bcall(**{which: None}) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(Lk=0), 2), (dict(Lq=(1 << 24) + 1), 2),
    (dict(D=96), 3), (dict(dtype=3), 4), (dict(scale=float("nan")), 5),
])
def test_bwd_bad_arguments(kw, code):
    assert bcall(**kw) == code


def test_bwd_misaligned_and_aliased():
    assert bcall(dout=DO + 8) == 6
    assert bcall(dk=DK + 2) == 6
    assert bcall(delta=DL + 2) == 6
    nbytes = 1 * 2 * 128 * 64 * 2
    assert bcall(dq=Q) == 7                   # dq on top of q
    assert bcall(dv=O + nbytes - 16) == 7     # dv overlapping the tail of o
    assert bcall(dk=DV + 64) == 7             # two outputs overlapping
    assert bcall(delta=L) == 7                # delta on top of lse
    assert bcall(delta=DQ + 16) == 7          # delta inside dq


def test_bwd_non_device_pointers_rejected_without_gpu():
    buf = [ctypes.create_string_buffer(1 << 16) for _ in range(10)]
    a = [((ctypes.addressof(b) + 15) // 16) * 16 for b in buf]
    assert bcall(*a) == 8


def test_bwd_kernel_selection():
    assert fa.fa_bwd_kernel_name(1, 2, 128, 128, 64, 1, 0.125, 0) == \
        "fa_bwd_valu_f32_d64_causal"
    assert fa.fa_bwd_kernel_name(1, 2, 128, 128, 65, 0, 1.0, 2) is None
    assert fa.fa_bwd_kernel_name(1, 2, 128, 0, 64, 0, 1.0, 2) is None


# ---- fa_fwd_ex: strides and window, host-side validation ------------------

def contig(B, H, L, D):
    return [H * L * D, L * D, D]


def xcall(strides=None, q=Q, k=K, v=V, o=O, lse=L, wl=-1, wr=-1, **kw):
    a = dict(GOOD)
    a.update(kw)
    if strides is None:
        sq = contig(a["B"], a["H"], a["Lq"], a["D"])
        sk = contig(a["B"], a["H"], a["Lk"], a["D"])
        strides = sq + sk + sk + sq
    return fa.fa_fwd_ex(q, k, v, o, lse, a["B"], a["H"], a["Lq"], a["Lk"],
                        a["D"], strides, a["causal"], wl, wr, a["scale"],
                        a["dtype"], None)


def test_ex_null_strides():
    assert fa.fa_fwd_ex(Q, K, V, O, L, 1, 2, 128, 128, 64, None, 0, -1, -1,
                        0.125, 2, None) == 1


def test_ex_bad_strides():
    base = contig(1, 2, 128, 64) * 4
    for i in range(12):
        s = list(base)
        s[i] = -8
        assert xcall(s) == 10, i
    s = list(base)
    s[2] = 1 << 25                       # row stride past 2^24
    assert xcall(s) == 10
    s = list(base)
    s[9:12] = [0, 0, 64]                 # o: every (b, h) on the same rows
    assert xcall(s) == 10
    s = list(base)
    s[11] = 32                           # o rows overlap (row stride < D)
    assert xcall(s) == 10
    s = list(base)
    s[5] = 68                            # k row stride not a multiple of 8
    assert xcall(s) == 6


def test_ex_layouts_pass_validation_until_device_check():
    # [B, L, H, D] strides are valid; the fake addresses then fail the
    # device-pointer check (8), i.e. every earlier check passed
    B, H, L, D = 2, 4, 128, 64
    blhd = [L * H * D, D, H * D]
    assert xcall(blhd * 4, B=B, H=H, Lq=L, Lk=L, D=D) == 8
    # packed QKV: q, k, v interleaved in one [B, L, 3, H, D] buffer
    pk = [L * 3 * H * D, D, 3 * H * D]
    assert xcall(pk * 3 + blhd, q=Q, k=Q + 2 * H * D, v=Q + 4 * H * D,
                 B=B, H=H, Lq=L, Lk=L, D=D) == 8
    assert xcall(wl=3, wr=0, causal=1) == 8


def test_ex_output_overlapping_input_rejected():
    nbytes = 1 * 2 * 128 * 64 * 2
    assert xcall(o=Q + 16) == 7
    assert xcall(o=K + nbytes - 16) == 7
    assert xcall(lse=O) == 7


def test_bwd_ex_validation():
    B, H, N, D = 1, 2, 128, 64
    st = contig(B, H, N, D) * 8

    def call(strides):
        return fa.fa_bwd_ex(Q, K, V, O, L, DO, DQ, DK, DV, DL, B, H, N, N, D,
                            strides, 0, -1, -1, 0.125, 2, None)
    assert fa.fa_bwd_ex(Q, K, V, O, L, DO, DQ, DK, DV, DL, B, H, N, N, D, None, 0,
                        -1, -1, 0.125, 2, None) == 1
    assert call(st) == 8                       # valid; fake addresses fail last
    bad = list(st)
    bad[3 * 5 + 2] = 32                        # dq rows overlap
    assert call(bad) == 10
    bad = list(st)
    bad[3 * 6 + 1] = -64                       # negative dk head stride
    assert call(bad) == 10
    bad = list(st)
    bad[3 * 4 + 2] = 68                        # dout row stride not 16-byte
    assert call(bad) == 6


def test_noalloc_rejects_sizes_past_its_scratch_without_touching_a_device():
    # B*H*Lq beyond the fixed scratch: FA_ERR_SCRATCH before any HIP call
    p = [(i + 1) << 40 for i in range(9)]
    Lq = (1 << 21) // 2 + 1
    rc = fa.fa_bwd_noalloc(*p, 1, 2, Lq, 64, 64, 0, 0.125, 2, None)
    assert rc == 11 and _lib.STATUS[rc] == "FA_ERR_SCRATCH"
    # the other checks come first, as in fa_bwd
    assert fa.fa_bwd_noalloc(*p[:8], None, 1, 2, 64, 64, 64, 0, 0.125, 2, None) == 1
    assert fa.fa_bwd_noalloc(*p, 1, 2, 64, 64, 96, 0, 0.125, 2, None) == 3
    assert fa.FA_NOALLOC_MAX_ROWS == 1 << 21
    text = open(HEADER).read()
    assert re.search(r"FA_NOALLOC_MAX_ROWS\s+\(1LL << 21\)", text)
