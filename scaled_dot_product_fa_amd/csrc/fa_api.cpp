// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation and
// kernel dispatch.  Every check runs on the host before anything is enqueued.
//
// The checks play the role of the asserts in the FlashAttention-2 forward
// article's host wrapper (inputs must be device tensors; shapes read from
// [B, H, L, D]); the output and the [B, H, Lq] fp32 row statistic are
// allocated by the caller, as the wrapper allocates them before its launch.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

// Fixed device scratch of fa_bwd_noalloc: the per-row statistic delta (fp32
// [B, H, Lq]) of up to FA_NOALLOC_MAX_ROWS rows, 8 MiB.  Each device holds
// its own copy until the process ends.  In host code this name is not a
// device address: kernels and copies take the per-device address that
// noalloc_scratch() obtains with hipGetSymbolAddress.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

namespace {

// Device address of `scratch` on `device` (the current device), looked up
// once per device and kept.  FA_OK, or FA_ERR_LAUNCH if the runtime cannot
// resolve the symbol.
int noalloc_scratch(int device, float **out)
{
    static std::mutex mu;
    static std::map<int, float *> ptrs;
    std::lock_guard<std::mutex> lock(mu);
    auto it = ptrs.find(device);
    if (it == ptrs.end()) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return FA_ERR_LAUNCH;
        }
        it = ptrs.emplace(device, static_cast<float *>(p)).first;
    }
    *out = it->second;
    return FA_OK;
}

bool overlaps(const void *a, int64_t an, const void *b, int64_t bn)
{
    if (a == nullptr || b == nullptr || an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// Shape, head dimension, dtype and scale checks (pure host logic).
int check_args(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, float scale,
               int dtype)
{
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
    if (Lq > FA_MAX_SEQ || Lk > FA_MAX_SEQ || B > FA_MAX_HEADS || H > FA_MAX_HEADS ||
        B * H > FA_MAX_HEADS)
        return FA_ERR_SHAPE;
    // grid size: B*H*ceil(Lq/32) workgroups must fit a 31-bit launch
    if (B * H * ((Lq + 31) / 32) > (int64_t)0x7fffffff) return FA_ERR_SHAPE;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    return FA_OK;
}

// Device memory of the current device (or managed memory)?
bool is_device_ptr(const void *p, int device)
{
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // do not leave a stale error behind
        return false;
    }
    if (attr.type == hipMemoryTypeManaged) return true;
    return attr.type == hipMemoryTypeDevice && attr.device == device;
}

int launch_forward(const fa::FwdArgs &a);

fa::FwdArgs make_args(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, int causal,
                      float scale, int dtype, void *stream)
{
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Lq = Lq;
    a.Lk = Lk;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.dtype = dtype;
    a.stream = static_cast<hipStream_t>(stream);
    // contiguous [B, H, L, D]
    const int64_t qs[3] = {H * Lq * D, Lq * D, D}, ks[3] = {H * Lk * D, Lk * D, D};
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = qs[i];
        a.os[i] = qs[i];
        a.ks[i] = ks[i];
        a.vs[i] = ks[i];
    }
    a.wl = -1;
    a.wr = -1;
    a.general = false;
    return a;
}

// Byte length of a strided [B, H, L, D] view (D contiguous) from its base.
int64_t view_bytes(int64_t B, int64_t H, int64_t L, int64_t D, const int64_t *s, int64_t es)
{
    return ((B - 1) * s[0] + (H - 1) * s[1] + (L - 1) * s[2] + D) * es;
}

// No two elements of the view share an address: with the dimensions in
// increasing stride order (D first, stride 1), every stride of a dimension
// longer than one is at least the span of the smaller dimensions.
bool view_injective(int64_t B, int64_t H, int64_t L, int64_t D, const int64_t *s)
{
    int64_t st[3] = {s[0], s[1], s[2]}, sz[3] = {B, H, L};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                int64_t t = st[i];
                st[i] = st[j];
                st[j] = t;
                t = sz[i];
                sz[i] = sz[j];
                sz[j] = t;
            }
    int64_t span = D;
    for (int i = 0; i < 3; ++i) {
        if (sz[i] == 1) continue;
        if (st[i] < span) return false;
        span = st[i] * (sz[i] - 1) + span;
    }
    return true;
}

// The contiguous strides of a [B, H, L, D] tensor (dimensions of length one
// may carry any stride).
bool is_contiguous(int64_t B, int64_t H, int64_t L, int64_t D, const int64_t *s)
{
    return (B == 1 || s[0] == H * L * D) && (H == 1 || s[1] == L * D) && (L == 1 || s[2] == D);
}

// Tuning override "NWxQBxBNxOCCxPIPE" (for sweeps), or "valu" to force the
// vector-ALU kernel.  Unset means the built-in choice.
bool env_tile(fa::MfmaTile &t, bool &force_valu)
{
    force_valu = false;
    const char *s = getenv("FA_TILE");
    if (s == nullptr || *s == '\0') return false;
    if (strcmp(s, "valu") == 0) {
        force_valu = true;
        return false;
    }
    int nw = 0, qb = 0, bn = 0, occ = 0, pipe = 0;
    char x1 = 0, x2 = 0, x3 = 0, x4 = 0;
    char tail = 0;
    const int n = sscanf(s, "%d%c%d%c%d%c%d%c%d%c", &nw, &x1, &qb, &x2, &bn, &x3, &occ, &x4,
                         &pipe, &tail);
    if (n != 9 || x1 != 'x' || x2 != 'x' || x3 != 'x' || x4 != 'x') return false;
    t = fa::MfmaTile{nw, qb, bn, occ, pipe};
    return true;
}

// Kernel choice for a validated forward call.
int launch_forward(const fa::FwdArgs &a)
{
    fa::MfmaTile tile{};
    bool force_valu = false;
    const bool have_tile = env_tile(tile, force_valu);
    hipError_t e;
    if (force_valu || !fa::mfma_supported(a))
        e = fa::valu_launch(a);
    else if (a.general)
        e = fa::mfma_launch_general(a);
    else
        e = fa::mfma_launch(a, have_tile ? tile : fa::mfma_choose_tile(a));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
           int64_t H, int64_t Lq, int64_t Lk, int64_t D, int causal, float scale, int dtype,
           void *stream)
{
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULL;
    int rc = check_args(B, H, Lq, Lk, D, scale, dtype);
    if (rc != FA_OK) return rc;

    const int64_t es = dtype == FA_F32 ? 4 : 2;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
    if ((mis & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;

    const int64_t nq = B * H * Lq * D * es, nk = B * H * Lk * D * es, nl = B * H * Lq * 4;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nk) || overlaps(o, nq, v, nk) ||
        overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
        overlaps(lse, nl, o, nq))
        return FA_ERR_ALIAS;

    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return FA_ERR_POINTER;
    }
    if (!is_device_ptr(q, device) || !is_device_ptr(k, device) || !is_device_ptr(v, device) ||
        !is_device_ptr(o, device) || (lse != nullptr && !is_device_ptr(lse, device)))
        return FA_ERR_POINTER;

    const fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype,
                                    stream);
    return launch_forward(a);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
              int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t *strides, int causal,
              int64_t window_left, int64_t window_right, float scale, int dtype, void *stream)
{
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || strides == nullptr)
        return FA_ERR_NULL;
    int rc = check_args(B, H, Lq, Lk, D, scale, dtype);
    if (rc != FA_OK) return rc;
    const int64_t es = dtype == FA_F32 ? 4 : 2;
    for (int i = 0; i < 12; ++i) {
        if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return FA_ERR_STRIDE;
        if (i % 3 == 2 && strides[i] > ((int64_t)1 << 24)) return FA_ERR_STRIDE;
    }
    const int64_t *qs = strides, *ks = strides + 3, *vs = strides + 6, *os = strides + 9;
    if (!view_injective(B, H, Lq, D, os)) return FA_ERR_STRIDE;
    for (int i = 0; i < 12; ++i)
        if ((strides[i] * es) % 16 != 0) return FA_ERR_ALIGN;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
    if ((mis & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;

    const int64_t nq = view_bytes(B, H, Lq, D, qs, es), nk = view_bytes(B, H, Lk, D, ks, es),
                  nv = view_bytes(B, H, Lk, D, vs, es), no = view_bytes(B, H, Lq, D, os, es),
                  nl = B * H * Lq * 4;
    if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv) ||
        overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nv) ||
        overlaps(lse, nl, o, no))
        return FA_ERR_ALIAS;

    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return FA_ERR_POINTER;
    }
    if (!is_device_ptr(q, device) || !is_device_ptr(k, device) || !is_device_ptr(v, device) ||
        !is_device_ptr(o, device) || (lse != nullptr && !is_device_ptr(lse, device)))
        return FA_ERR_POINTER;

    fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype, stream);
    // a window that cannot exclude any key is no window
    a.wl = (window_left < 0 || window_left >= Lq + Lk) ? -1 : (int)window_left;
    a.wr = (window_right < 0 || window_right >= Lq + Lk) ? -1 : (int)window_right;
    const bool contiguous = is_contiguous(B, H, Lq, D, qs) && is_contiguous(B, H, Lk, D, ks) &&
                            is_contiguous(B, H, Lk, D, vs) && is_contiguous(B, H, Lq, D, os);
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = qs[i];
        a.ks[i] = ks[i];
        a.vs[i] = vs[i];
        a.os[i] = os[i];
    }
    a.general = !contiguous || a.wl >= 0 || a.wr >= 0;
    return launch_forward(a);
}

}  // extern "C"

namespace {

// Validation and launch shared by fa_bwd, fa_bwd_ex and fa_bwd_noalloc.
// strides: 24 values (batch, head, row) of q, k, v, o, dout, dq, dk, dv.
// delta_internal: delta is the library's own scratch (not a caller buffer,
// so it is not checked as one).
int bwd_common(const void *q, const void *k, const void *v, const void *o, const float *lse,
               const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
               int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t *strides, int causal,
               int64_t window_left, int64_t window_right, float scale, int dtype, void *stream,
               bool delta_internal = false)
{
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
        dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || delta == nullptr)
        return FA_ERR_NULL;
    int rc = check_args(B, H, Lq, Lk, D, scale, dtype);
    if (rc != FA_OK) return rc;
    // the key-block grid B*H*ceil(Lk/32) must fit a 31-bit launch as well
    if (B * H * ((Lk + 31) / 32) > (int64_t)0x7fffffff) return FA_ERR_SHAPE;
    const int64_t es = dtype == FA_F32 ? 4 : 2;
    const int64_t L[8] = {Lq, Lk, Lk, Lq, Lq, Lq, Lk, Lk};
    for (int i = 0; i < 24; ++i) {
        if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return FA_ERR_STRIDE;
        if (i % 3 == 2 && strides[i] > ((int64_t)1 << 24)) return FA_ERR_STRIDE;
    }
    for (int t = fa::kDq; t <= fa::kDv; ++t)
        if (!view_injective(B, H, L[t], D, strides + 3 * t)) return FA_ERR_STRIDE;
    for (int i = 0; i < 24; ++i)
        if ((strides[i] * es) % 16 != 0) return FA_ERR_ALIGN;

    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                          reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                          reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
    if ((mis & 15u) != 0 ||
        ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(delta)) & 3u) != 0)
        return FA_ERR_ALIGN;

    int64_t n[8];
    for (int t = 0; t < 8; ++t) n[t] = view_bytes(B, H, L[t], D, strides + 3 * t, es);
    const int64_t nl = B * H * Lq * 4;
    // outputs dq, dk, dv, delta against the inputs and each other
    const void *ins[6] = {q, k, v, o, lse, dout};
    const int64_t in_n[6] = {n[fa::kQ], n[fa::kK], n[fa::kV], n[fa::kO], nl, n[fa::kDout]};
    void *outs[4] = {dq, dk, dv, delta};
    const int64_t out_n[4] = {n[fa::kDq], n[fa::kDk], n[fa::kDv], nl};
    for (int w = 0; w < 4; ++w) {
        for (int r = 0; r < 6; ++r)
            if (overlaps(outs[w], out_n[w], ins[r], in_n[r])) return FA_ERR_ALIAS;
        for (int u = w + 1; u < 4; ++u)
            if (overlaps(outs[w], out_n[w], outs[u], out_n[u])) return FA_ERR_ALIAS;
    }

    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return FA_ERR_POINTER;
    }
    for (int r = 0; r < 6; ++r)
        if (!is_device_ptr(ins[r], device)) return FA_ERR_POINTER;
    for (int w = 0; w < (delta_internal ? 3 : 4); ++w)
        if (!is_device_ptr(outs[w], device)) return FA_ERR_POINTER;

    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.B = B;
    a.H = H;
    a.Lq = Lq;
    a.Lk = Lk;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.dtype = dtype;
    a.stream = static_cast<hipStream_t>(stream);
    bool contiguous = true;
    for (int t = 0; t < 8; ++t) {
        for (int i = 0; i < 3; ++i) a.st[t][i] = strides[3 * t + i];
        contiguous = contiguous && is_contiguous(B, H, L[t], D, strides + 3 * t);
    }
    a.wl = (window_left < 0 || window_left >= Lq + Lk) ? -1 : (int)window_left;
    a.wr = (window_right < 0 || window_right >= Lq + Lk) ? -1 : (int)window_right;
    a.general = !contiguous || a.wl >= 0 || a.wr >= 0;
    fa::MfmaTile unused{};
    bool force_valu = false;
    (void)env_tile(unused, force_valu);
    hipError_t e = fa::bwd_delta_launch(a);
    if (e == hipSuccess)
        e = (!force_valu && fa::bwd_mfma_supported(a)) ? fa::bwd_mfma_launch(a)
                                                        : fa::bwd_valu_launch(a);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B, int64_t H,
           int64_t Lq, int64_t Lk, int64_t D, int causal, float scale, int dtype, void *stream)
{
    const int64_t sq[3] = {H * Lq * D, Lq * D, D}, sk[3] = {H * Lk * D, Lk * D, D};
    int64_t st[24];
    const int64_t *per[8] = {sq, sk, sk, sq, sq, sq, sk, sk};
    for (int t = 0; t < 8; ++t)
        for (int i = 0; i < 3; ++i) st[3 * t + i] = per[t][i];
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Lq, Lk, D, st, causal,
                      -1, -1, scale, dtype, stream);
}

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const float *lse, const void *dout, void *dq, void *dk, void *dv, int64_t B,
                   int64_t H, int64_t Lq, int64_t Lk, int64_t D, int causal, float scale,
                   int dtype, void *stream)
{
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
        dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return FA_ERR_NULL;
    int rc = check_args(B, H, Lq, Lk, D, scale, dtype);
    if (rc != FA_OK) return rc;
    if (B * H * Lq > FA_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return FA_ERR_POINTER;
    }
    float *ws = nullptr;
    rc = noalloc_scratch(device, &ws);
    if (rc != FA_OK) return rc;
    const int64_t sq[3] = {H * Lq * D, Lq * D, D}, sk[3] = {H * Lk * D, Lk * D, D};
    int64_t st[24];
    const int64_t *per[8] = {sq, sk, sk, sq, sq, sq, sk, sk};
    for (int t = 0; t < 8; ++t)
        for (int i = 0; i < 3; ++i) st[3 * t + i] = per[t][i];
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, Lq, Lk, D, st, causal, -1,
                      -1, scale, dtype, stream, true);
}

int fa_bwd_ex(const void *q, const void *k, const void *v, const void *o, const float *lse,
              const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
              int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t *strides, int causal,
              int64_t window_left, int64_t window_right, float scale, int dtype, void *stream)
{
    if (strides == nullptr) return FA_ERR_NULL;
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Lq, Lk, D, strides,
                      causal, window_left, window_right, scale, dtype, stream);
}

const char *fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H, Lq or Lk out of range";
    case FA_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_F32, FA_F16 or FA_BF16";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGN: return "tensors must be 16-byte aligned, lse and delta 4-byte aligned";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_POINTER: return "a pointer is not device memory of the current device";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_STRIDE: return "a stride is negative or too large, or o has overlapping elements";
    case FA_ERR_SCRATCH:
        return "B*H*Lq exceeds the fixed scratch of fa_bwd_noalloc (FA_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
    }
}

const char *fa_kernel_name(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                           int causal, float scale, int dtype)
{
    if (check_args(B, H, Lq, Lk, D, scale, dtype) != FA_OK) return nullptr;
    const fa::FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, Lq, Lk,
                                    D, causal, scale, dtype, nullptr);
    fa::MfmaTile tile{};
    bool force_valu = false;
    const bool have_tile = env_tile(tile, force_valu);
    if (!force_valu && fa::mfma_supported(a))
        return fa::mfma_kernel_name(a, have_tile ? tile : fa::mfma_choose_tile(a));
    return fa::valu_kernel_name(a);
}

const char *fa_bwd_kernel_name(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                               int causal, float scale, int dtype)
{
    if (check_args(B, H, Lq, Lk, D, scale, dtype) != FA_OK) return nullptr;
    if (B * H * ((Lk + 31) / 32) > (int64_t)0x7fffffff) return nullptr;
    fa::BwdArgs a{};
    a.B = B;
    a.H = H;
    a.Lq = Lq;
    a.Lk = Lk;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.dtype = dtype;
    fa::MfmaTile unused{};
    bool force_valu = false;
    (void)env_tile(unused, force_valu);
    if (!force_valu && fa::bwd_mfma_supported(a)) return fa::bwd_mfma_kernel_name(a);
    return fa::bwd_valu_kernel_name(a);
}

int fa_version(void) { return 200; }

}  // extern "C"
