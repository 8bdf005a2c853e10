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
// streamed through LDS, as in the forward).  Serves fp32 I/O and every case
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

__device__ __forceinline__ float quad_sum(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

// delta_i = dO_i . O_i, one row per 4 threads.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_delta_kernel(
    const T *__restrict__ o, const T *__restrict__ dout, float *__restrict__ delta,
    int64_t rows)
{
    constexpr int DS = D / 4;
    const int64_t r = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 2);
    const int t4 = threadIdx.x & 3;
    float part = 0.f;
    if (r < rows) {
        const T *orow = o + r * D + t4 * DS;
        const T *grow = dout + r * D + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) part = fmaf(to_f32(orow[e]), to_f32(grow[e]), part);
    }
    part = quad_sum(part);
    if (r < rows && t4 == 0) delta[r] = part;
}

// dK, dV for 64 keys; query rows streamed in tiles of 32.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_bwd_dkdv_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ delta, T *__restrict__ dk, T *__restrict__ dv, int Lq, int Lk,
    float scale, int ntk)
{
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

    const T *qh = q + bh * (int64_t)Lq * D;
    const T *gh = dout + bh * (int64_t)Lq * D;
    const float *lh = lse + bh * (int64_t)Lq;
    const float *dh = delta + bh * (int64_t)Lq;

    float kr[DS], vr[DS], dka[DS], dva[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) {
        const int64_t off = (bh * Lk + kj) * (int64_t)D + t4 * DS + e;
        kr[e] = key_valid ? to_f32(k[off]) * scale : 0.f;
        vr[e] = key_valid ? to_f32(v[off]) : 0.f;
        dka[e] = 0.f;
        dva[e] = 0.f;
    }

    // causal: rows below the block's first key see none of its keys
    const int i_begin = CAUSAL ? (k_first / kTile) * kTile : 0;
    for (int i0 = i_begin; i0 < Lq; i0 += kTile) {
        __syncthreads();
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const int qi = i0 + r;
            qs[r][c] = qi < Lq ? to_f32(qh[(int64_t)qi * D + c]) : 0.f;
            gs[r][c] = qi < Lq ? to_f32(gh[(int64_t)qi * D + c]) : 0.f;
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
            const bool keep = key_valid && qi < Lq && (!CAUSAL || kj <= qi);
            const float p = keep ? expf(s - ls[r]) : 0.f;
            const float dsv = p * (dp - ds_[r]);
#pragma unroll
            for (int e = 0; e < DS; ++e) {
                dva[e] = fmaf(p, gs[r][t4 * DS + e], dva[e]);
                dka[e] = fmaf(dsv, qs[r][t4 * DS + e], dka[e]);
            }
        }
    }
    if (key_valid) {
        const int64_t off = (bh * Lk + kj) * (int64_t)D + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) {
            dk[off + e] = from_f32<T>(dka[e] * scale);
            dv[off + e] = from_f32<T>(dva[e]);
        }
    }
}

// dQ for 64 query rows; keys streamed in tiles of 32.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_bwd_dq_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ delta, T *__restrict__ dq, int Lq, int Lk, float scale, int ntq)
{
    constexpr int DS = D / 4;
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];

    const int tid = threadIdx.x;
    const int t4 = tid & 3;
    const int64_t bh = blockIdx.x / ntq;
    const int q_first = (blockIdx.x % ntq) * kRows;
    const int qi = q_first + (tid >> 2);
    const bool row_valid = qi < Lq;

    const T *kh = k + bh * (int64_t)Lk * D;
    const T *vh = v + bh * (int64_t)Lk * D;
    float qr[DS], gr[DS], acc[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) {
        const int64_t off = (bh * Lq + qi) * (int64_t)D + t4 * DS + e;
        qr[e] = row_valid ? to_f32(q[off]) * scale : 0.f;
        gr[e] = row_valid ? to_f32(dout[off]) : 0.f;
        acc[e] = 0.f;
    }
    const float lse_i = row_valid ? lse[bh * Lq + qi] : 0.f;
    const float delta_i = row_valid ? delta[bh * Lq + qi] : 0.f;

    const int kv_end = CAUSAL ? min(Lk, q_first + kRows) : Lk;
    for (int k0 = 0; k0 < kv_end; k0 += kTile) {
        __syncthreads();
        for (int idx = tid; idx < kTile * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const int kr = k0 + r;
            ks[r][c] = kr < Lk ? to_f32(kh[(int64_t)kr * D + c]) : 0.f;
            vs[r][c] = kr < Lk ? to_f32(vh[(int64_t)kr * D + c]) : 0.f;
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
            const bool keep = row_valid && kj < Lk && (!CAUSAL || kj <= qi);
            const float p = keep ? expf(s - lse_i) : 0.f;
            const float dsv = p * (dp - delta_i);
#pragma unroll
            for (int e = 0; e < DS; ++e) acc[e] = fmaf(dsv, ks[j][t4 * DS + e], acc[e]);
        }
    }
    if (row_valid) {
        T *row = dq + (bh * Lq + qi) * (int64_t)D + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) row[e] = from_f32<T>(acc[e] * scale);
    }
}

template <typename T, int D>
hipError_t delta_t(const BwdArgs &a)
{
    const int64_t rows = a.B * a.H * a.Lq;
    hipLaunchKernelGGL((fa_bwd_delta_kernel<T, D>), dim3((unsigned)((rows + kRows - 1) / kRows)),
                       dim3(kThreads), 0, a.stream, static_cast<const T *>(a.o),
                       static_cast<const T *>(a.dout), a.delta, rows);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t grads_t(const BwdArgs &a)
{
    const int ntk = (int)((a.Lk + kRows - 1) / kRows);
    hipLaunchKernelGGL((fa_bwd_dkdv_valu_kernel<T, D, CAUSAL>),
                       dim3((unsigned)(a.B * a.H * ntk)), dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<const T *>(a.dout), a.lse,
                       a.delta, static_cast<T *>(a.dk), static_cast<T *>(a.dv), (int)a.Lq,
                       (int)a.Lk, a.scale, ntk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntq = (int)((a.Lq + kRows - 1) / kRows);
    hipLaunchKernelGGL((fa_bwd_dq_valu_kernel<T, D, CAUSAL>),
                       dim3((unsigned)(a.B * a.H * ntq)), dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<const T *>(a.dout), a.lse,
                       a.delta, static_cast<T *>(a.dq), (int)a.Lq, (int)a.Lk, a.scale, ntq);
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
