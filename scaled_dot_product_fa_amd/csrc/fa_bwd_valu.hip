// fa_bwd_valu.hip -- attention backward on the vector ALUs (fp32 arithmetic).
//
// Gradients of O = softmax(scale Q K^T [+causal]) V for an incoming dO, by
// the chain rule through that definition, with the probabilities recomputed
// from the forward's row statistic instead of stored (the FlashAttention-2
// forward article keeps Q, K, V, O and the statistic for the backward and
// notes that the backward may recompute rather than store):
//
//   p_ij    = exp(scale q_i.k_j - lse_i)       (0 where masked)
//   delta_i = dO_i . O_i                       (= sum_j p_ij dp_ij)
//   dp_ij   = dO_i . v_j
//   ds_ij   = p_ij (dp_ij - delta_i)
//   dV_j    = sum_i p_ij dO_i
//   dK_j    = scale sum_i ds_ij q_i
//   dQ_i    = scale sum_j ds_ij k_j
//
// Three kernels and no atomics: delta per row; dK and dV per block of keys
// (query tiles streamed through LDS); dQ per block of query rows (key tiles
// streamed through LDS, as in the forward).  Tensors are addressed through
// (batch, head, row) element strides, and an optional local window narrows
// the rows (dK/dV) or keys (dQ) that are visited.  Serves fp32 I/O and every case
// the MFMA backward leaves out.  Layout as in the forward VALU kernel: 256
// threads = 64 rows x 4 threads, thread t4 of a row owning head-dimension
// slice [t4*D/4, (t4+1)*D/4); dot products are reduced over the 4 threads
// with lane shuffles.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 64;     // rows (queries or keys) owned per workgroup
constexpr int kTile = 32;     // rows per streamed LDS tile
constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

// What the kernels need of a backward call: pointers, sizes, the window and
// the element strides (batch, head, row) of q, k, v, o, dout, dq, dk, dv.
struct VParams {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    float *delta;
    void *dq, *dk, *dv;
    int H, Lq, Lk, wl, wr;
    int64_t rows;
    float scale;
    int64_t st[8][3];
};

__device__ __forceinline__ int64_t base_of(const VParams &p, int t, int64_t bh)
{
    return (bh / p.H) * p.st[t][0] + (bh % p.H) * p.st[t][1];
}

// visible keys of query row i: j in [lo, hi]
__device__ __forceinline__ bool keeps(const VParams &p, bool causal, int i, int j)
{
    return (!causal || j <= i) && (p.wl < 0 || j >= i - p.wl) && (p.wr < 0 || j <= i + p.wr);
}

__device__ __forceinline__ float quad_sum(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

// delta_i = dO_i . O_i, one row per 4 threads.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_delta_kernel(VParams p)
{
    constexpr int DS = D / 4;
    const int64_t rows = p.rows;
    float *__restrict__ delta = p.delta;
    const int64_t r = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 2);
    const int t4 = threadIdx.x & 3;
    float part = 0.f;
    if (r < rows) {
        const int64_t bh = r / p.Lq, i = r % p.Lq;
        const T *orow = static_cast<const T *>(p.o) + base_of(p, 3, bh) + i * p.st[3][2] + t4 * DS;
        const T *grow = static_cast<const T *>(p.dout) + base_of(p, 4, bh) + i * p.st[4][2] + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) part = fmaf(to_f32(orow[e]), to_f32(grow[e]), part);
    }
    part = quad_sum(part);
    if (r < rows && t4 == 0) delta[r] = part;
}

// dK, dV for 64 keys; query rows streamed in tiles of 32.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_bwd_dkdv_valu_kernel(VParams p, int ntk)
{
    const int Lq = p.Lq, Lk = p.Lk;
    const float scale = p.scale;
    const float *__restrict__ lse = p.lse;
    const float *__restrict__ delta = p.delta;
    constexpr int DS = D / 4;
    __shared__ float qs[kTile][D];
    __shared__ float gs[kTile][D];
    __shared__ float ls[kTile], ds_[kTile];

    const int tid = threadIdx.x;
    const int t4 = tid & 3;
    const int64_t bh = blockIdx.x / ntk;
    const int k_first = (blockIdx.x % ntk) * kRows;
    const int kj = k_first + (tid >> 2);
    const bool key_valid = kj < Lk;

    const T *qh = static_cast<const T *>(p.q) + base_of(p, 0, bh);
    const T *gh = static_cast<const T *>(p.dout) + base_of(p, 4, bh);
    const T *kh = static_cast<const T *>(p.k) + base_of(p, 1, bh);
    const T *vh = static_cast<const T *>(p.v) + base_of(p, 2, bh);
    const int64_t q_sl = p.st[0][2], g_sl = p.st[4][2];
    const float *lh = lse + bh * (int64_t)Lq;
    const float *dh = delta + bh * (int64_t)Lq;

    float kr[DS], vr[DS], dka[DS], dva[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) {
        kr[e] = key_valid ? to_f32(kh[(int64_t)kj * p.st[1][2] + t4 * DS + e]) * scale : 0.f;
        vr[e] = key_valid ? to_f32(vh[(int64_t)kj * p.st[2][2] + t4 * DS + e]) : 0.f;
        dka[e] = 0.f;
        dva[e] = 0.f;
    }

    // rows that can see a key of the block: causal rows from its first key,
    // window rows from first key - wr to last key + wl
    int i_begin = CAUSAL ? (k_first / kTile) * kTile : 0;
    int i_end = Lq;
    if (p.wr >= 0) i_begin = max(i_begin, max(0, k_first - p.wr) / kTile * kTile);
    if (p.wl >= 0) i_end = min(Lq, k_first + kRows + p.wl);
    for (int i0 = i_begin; i0 < i_end; i0 += kTile) {
        __syncthreads();
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const int qi = i0 + r;
            qs[r][c] = qi < Lq ? to_f32(qh[(int64_t)qi * q_sl + c]) : 0.f;
            gs[r][c] = qi < Lq ? to_f32(gh[(int64_t)qi * g_sl + c]) : 0.f;
        }
        if (tid < kTile) {
            const int qi = i0 + tid;
            ls[tid] = qi < Lq ? lh[qi] : 0.f;
            ds_[tid] = qi < Lq ? dh[qi] : 0.f;
        }
        __syncthreads();
#pragma unroll 2
        for (int r = 0; r < kTile; ++r) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < DS; ++e) {
                s = fmaf(kr[e], qs[r][t4 * DS + e], s);
                dp = fmaf(vr[e], gs[r][t4 * DS + e], dp);
            }
            s = quad_sum(s);
            dp = quad_sum(dp);
            const int qi = i0 + r;
            const bool keep = key_valid && qi < Lq && keeps(p, CAUSAL, qi, kj);
            const float pr = keep ? expf(s - ls[r]) : 0.f;
            const float dsv = pr * (dp - ds_[r]);
#pragma unroll
            for (int e = 0; e < DS; ++e) {
                dva[e] = fmaf(pr, gs[r][t4 * DS + e], dva[e]);
                dka[e] = fmaf(dsv, qs[r][t4 * DS + e], dka[e]);
            }
        }
    }
    if (key_valid) {
        T *dkr = static_cast<T *>(p.dk) + base_of(p, 6, bh) + (int64_t)kj * p.st[6][2] + t4 * DS;
        T *dvr = static_cast<T *>(p.dv) + base_of(p, 7, bh) + (int64_t)kj * p.st[7][2] + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) {
            dkr[e] = from_f32<T>(dka[e] * scale);
            dvr[e] = from_f32<T>(dva[e]);
        }
    }
}

// dQ for 64 query rows; keys streamed in tiles of 32.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_bwd_dq_valu_kernel(VParams p, int ntq)
{
    const int Lq = p.Lq, Lk = p.Lk;
    const float scale = p.scale;
    const float *__restrict__ lse = p.lse;
    const float *__restrict__ delta = p.delta;
    constexpr int DS = D / 4;
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];

    const int tid = threadIdx.x;
    const int t4 = tid & 3;
    const int64_t bh = blockIdx.x / ntq;
    const int q_first = (blockIdx.x % ntq) * kRows;
    const int qi = q_first + (tid >> 2);
    const bool row_valid = qi < Lq;

    const T *kh = static_cast<const T *>(p.k) + base_of(p, 1, bh);
    const T *vh = static_cast<const T *>(p.v) + base_of(p, 2, bh);
    const int64_t k_sl = p.st[1][2], v_sl = p.st[2][2];
    const T *qrow = static_cast<const T *>(p.q) + base_of(p, 0, bh) + (int64_t)qi * p.st[0][2];
    const T *grow = static_cast<const T *>(p.dout) + base_of(p, 4, bh) + (int64_t)qi * p.st[4][2];
    float qr[DS], gr[DS], acc[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) {
        qr[e] = row_valid ? to_f32(qrow[t4 * DS + e]) * scale : 0.f;
        gr[e] = row_valid ? to_f32(grow[t4 * DS + e]) : 0.f;
        acc[e] = 0.f;
    }
    const float lse_i = row_valid ? lse[bh * Lq + qi] : 0.f;
    const float delta_i = row_valid ? delta[bh * Lq + qi] : 0.f;

    int kv_end = CAUSAL ? min(Lk, q_first + kRows) : Lk;
    int kv_begin = 0;
    if (p.wl >= 0) kv_begin = max(0, q_first - p.wl) / kTile * kTile;
    if (p.wr >= 0) kv_end = min(kv_end, q_first + kRows + p.wr);
    for (int k0 = kv_begin; k0 < kv_end; k0 += kTile) {
        __syncthreads();
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const int kr = k0 + r;
            ks[r][c] = kr < Lk ? to_f32(kh[(int64_t)kr * k_sl + c]) : 0.f;
            vs[r][c] = kr < Lk ? to_f32(vh[(int64_t)kr * v_sl + c]) : 0.f;
        }
        __syncthreads();
#pragma unroll 2
        for (int j = 0; j < kTile; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < DS; ++e) {
                s = fmaf(qr[e], ks[j][t4 * DS + e], s);
                dp = fmaf(gr[e], vs[j][t4 * DS + e], dp);
            }
            s = quad_sum(s);
            dp = quad_sum(dp);
            const int kj = k0 + j;
            const bool keep = row_valid && kj < Lk && keeps(p, CAUSAL, qi, kj);
            const float pr = keep ? expf(s - lse_i) : 0.f;
            const float dsv = pr * (dp - delta_i);
#pragma unroll
            for (int e = 0; e < DS; ++e) acc[e] = fmaf(dsv, ks[j][t4 * DS + e], acc[e]);
        }
    }
    if (row_valid) {
        T *row = static_cast<T *>(p.dq) + base_of(p, 5, bh) + (int64_t)qi * p.st[5][2] + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) row[e] = from_f32<T>(acc[e] * scale);
    }
}

VParams make_params(const BwdArgs &a)
{
    VParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.dout = a.dout;
    p.lse = a.lse;
    p.delta = a.delta;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.H = (int)a.H;
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.wl = a.wl;
    p.wr = a.wr;
    p.rows = a.B * a.H * a.Lq;
    p.scale = a.scale;
    for (int t = 0; t < 8; ++t)
        for (int i = 0; i < 3; ++i) p.st[t][i] = a.st[t][i];
    return p;
}

template <typename T, int D>
hipError_t delta_t(const BwdArgs &a)
{
    const VParams p = make_params(a);
    hipLaunchKernelGGL((fa_bwd_delta_kernel<T, D>), dim3((unsigned)((p.rows + kRows - 1) / kRows)),
                       dim3(kThreads), 0, a.stream, p);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t grads_t(const BwdArgs &a)
{
    const VParams p = make_params(a);
    const int ntk = (int)((a.Lk + kRows - 1) / kRows);
    hipLaunchKernelGGL((fa_bwd_dkdv_valu_kernel<T, D, CAUSAL>),
                       dim3((unsigned)(a.B * a.H * ntk)), dim3(kThreads), 0, a.stream, p, ntk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntq = (int)((a.Lq + kRows - 1) / kRows);
    hipLaunchKernelGGL((fa_bwd_dq_valu_kernel<T, D, CAUSAL>),
                       dim3((unsigned)(a.B * a.H * ntq)), dim3(kThreads), 0, a.stream, p, ntq);
    return hipGetLastError();
}

template <typename T>
hipError_t delta_dtype(const BwdArgs &a)
{
    return a.D == 64 ? delta_t<T, 64>(a) : delta_t<T, 128>(a);
}

template <typename T>
hipError_t grads_dtype(const BwdArgs &a)
{
    if (a.D == 64) return a.causal ? grads_t<T, 64, true>(a) : grads_t<T, 64, false>(a);
    return a.causal ? grads_t<T, 128, true>(a) : grads_t<T, 128, false>(a);
}

}  // namespace

hipError_t bwd_delta_launch(const BwdArgs &a)
{
    switch (a.dtype) {
    case 0: return delta_dtype<float>(a);
    case 1: return delta_dtype<_Float16>(a);
    default: return delta_dtype<__bf16>(a);
    }
}

hipError_t bwd_valu_launch(const BwdArgs &a)
{
    switch (a.dtype) {
    case 0: return grads_dtype<float>(a);
    case 1: return grads_dtype<_Float16>(a);
    default: return grads_dtype<__bf16>(a);
    }
}

const char *bwd_valu_kernel_name(const BwdArgs &a)
{
    static const char *names[3][2][2] = {
        {{"fa_bwd_valu_f32_d64", "fa_bwd_valu_f32_d64_causal"},
         {"fa_bwd_valu_f32_d128", "fa_bwd_valu_f32_d128_causal"}},
        {{"fa_bwd_valu_f16_d64", "fa_bwd_valu_f16_d64_causal"},
         {"fa_bwd_valu_f16_d128", "fa_bwd_valu_f16_d128_causal"}},
        {{"fa_bwd_valu_bf16_d64", "fa_bwd_valu_bf16_d64_causal"},
         {"fa_bwd_valu_bf16_d128", "fa_bwd_valu_bf16_d128_causal"}},
    };
    return names[a.dtype][a.D == 128][a.causal ? 1 : 0];
}

}  // namespace fa
