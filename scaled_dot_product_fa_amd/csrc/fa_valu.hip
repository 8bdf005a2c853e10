// fa_valu.hip -- attention forward on the vector ALUs (fp32 arithmetic).
//
// Serves fp32 I/O (fp32 products and sums throughout, so the result stays
// within fp32 rounding of the exact value) and the cases the MFMA kernel
// leaves out (scale <= 0).  Same method as the MFMA kernel: one workgroup per
// block of query rows, K/V streamed through LDS in tiles, online softmax
// (running max m, running sum l, unnormalised accumulator, rescale factor
// exp(m_old - m_new)) as in the FlashAttention-2 forward article
// (_attn_fwd_inner) and "Triton Ascend Attention" (online softmax section);
// causal tiles past the diagonal of the block are never loaded.
//
// Layout: 256 threads = 64 query rows x 4 threads; thread t4 of a row owns
// head-dimension slice [t4*D/4, (t4+1)*D/4).  Scores are reduced across the
// 4 threads of a row with lane shuffles.  Tensors are addressed through
// (batch, head, row) element strides, so strided views work as they are;
// an optional local window (keys i - wl .. i + wr) narrows the key range.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kValuBM = 64;    // query rows per workgroup
constexpr int kValuBN = 32;    // keys per K/V tile
constexpr int kValuThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

struct ValuParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int H, Lq, Lk, ntq, wl, wr;
    float scale;
    int64_t qs[3], ks[3], vs[3], os[3];
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kValuThreads) void fa_fwd_valu_kernel(ValuParams p)
{
    const int Lq = p.Lq, Lk = p.Lk, ntq = p.ntq;
    const float scale = p.scale;
    float *__restrict__ lse = p.lse;
    constexpr int DS = D / 4;  // dims owned by one thread
    __shared__ float ks[kValuBN][D];
    __shared__ float vs[kValuBN][D];

    const int tid = threadIdx.x;
    const int row_local = tid >> 2;
    const int t4 = tid & 3;
    const int64_t bh = blockIdx.x / ntq;
    const int qt = blockIdx.x % ntq;
    const int q_first = qt * kValuBM;
    const int qi = q_first + row_local;
    const bool row_valid = qi < Lq;

    const int64_t b_ = bh / p.H, h_ = bh % p.H;
    const T *qh = static_cast<const T *>(p.q) + b_ * p.qs[0] + h_ * p.qs[1];
    const T *kh = static_cast<const T *>(p.k) + b_ * p.ks[0] + h_ * p.ks[1];
    const T *vh = static_cast<const T *>(p.v) + b_ * p.vs[0] + h_ * p.vs[1];
    T *oh = static_cast<T *>(p.o) + b_ * p.os[0] + h_ * p.os[1];
    const int64_t q_sl = p.qs[2], k_sl = p.ks[2], v_sl = p.vs[2], o_sl = p.os[2];

    float qr[DS], acc[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) {
        qr[e] = row_valid ? to_f32(qh[(int64_t)qi * q_sl + t4 * DS + e]) : 0.f;
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    int kv_end = CAUSAL ? min(Lk, q_first + kValuBM) : Lk;
    int kv_begin = 0;
    if (p.wl >= 0) kv_begin = max(0, q_first - p.wl) / kValuBN * kValuBN;
    if (p.wr >= 0) kv_end = min(kv_end, q_first + kValuBM + p.wr);
    for (int k0 = kv_begin; k0 < kv_end; k0 += kValuBN) {
        __syncthreads();
        for (int idx = tid; idx < kValuBN * D; idx += kValuThreads) {
            const int r = idx / D, c = idx % D;
            const int kr = k0 + r;
            ks[r][c] = kr < Lk ? to_f32(kh[(int64_t)kr * k_sl + c]) : 0.f;
            vs[r][c] = kr < Lk ? to_f32(vh[(int64_t)kr * v_sl + c]) : 0.f;
        }
        __syncthreads();

        float s[kValuBN];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < kValuBN; ++j) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < DS; ++e) part = fmaf(qr[e], ks[j][t4 * DS + e], part);
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            const int kj = k0 + j;
            const bool keep = kj < Lk && (!CAUSAL || kj <= qi) &&
                              (p.wl < 0 || kj >= qi - p.wl) && (p.wr < 0 || kj <= qi + p.wr);
            s[j] = keep ? part * scale : -INFINITY;
            tmax = fmaxf(tmax, s[j]);
        }
        const float m_new = fmaxf(m, tmax);
        // a row with no visible key so far keeps m = -inf; use 0 as the
        // reference then so that exp(-inf - ref) = 0 instead of NaN
        const float ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = expf(m - ref);
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] *= alpha;
#pragma unroll
        for (int j = 0; j < kValuBN; ++j) {
            const float p = expf(s[j] - ref);
            psum += p;
#pragma unroll
            for (int e = 0; e < DS; ++e) acc[e] = fmaf(p, vs[j][t4 * DS + e], acc[e]);
        }
        l = l * alpha + psum;
        m = m_new;
    }

    if (row_valid) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        T *orow = oh + (int64_t)qi * o_sl + t4 * DS;
#pragma unroll
        for (int e = 0; e < DS; ++e) orow[e] = from_f32<T>(acc[e] * inv);
        if (lse != nullptr && t4 == 0)
            lse[bh * (int64_t)Lq + qi] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const FwdArgs &a)
{
    ValuParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.H = (int)a.H;
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + kValuBM - 1) / kValuBM);
    p.wl = a.wl;
    p.wr = a.wr;
    p.scale = a.scale;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = a.qs[i];
        p.ks[i] = a.ks[i];
        p.vs[i] = a.vs[i];
        p.os[i] = a.os[i];
    }
    const int64_t nwg = a.B * a.H * p.ntq;
    hipLaunchKernelGGL((fa_fwd_valu_kernel<T, D, CAUSAL>), dim3((unsigned)nwg),
                       dim3(kValuThreads), 0, a.stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const FwdArgs &a)
{
    if (a.D == 64)
        return a.causal ? launch_t<T, 64, true>(a) : launch_t<T, 64, false>(a);
    return a.causal ? launch_t<T, 128, true>(a) : launch_t<T, 128, false>(a);
}

}  // namespace

const char *valu_kernel_name(const FwdArgs &a)
{
    static const char *names[3][2][2] = {
        {{"fa_fwd_valu_f32_d64", "fa_fwd_valu_f32_d64_causal"},
         {"fa_fwd_valu_f32_d128", "fa_fwd_valu_f32_d128_causal"}},
        {{"fa_fwd_valu_f16_d64", "fa_fwd_valu_f16_d64_causal"},
         {"fa_fwd_valu_f16_d128", "fa_fwd_valu_f16_d128_causal"}},
        {{"fa_fwd_valu_bf16_d64", "fa_fwd_valu_bf16_d64_causal"},
         {"fa_fwd_valu_bf16_d128", "fa_fwd_valu_bf16_d128_causal"}},
    };
    return names[a.dtype][a.D == 128][a.causal ? 1 : 0];
}

hipError_t valu_launch(const FwdArgs &a)
{
    switch (a.dtype) {
    case 0: return launch_dtype<float>(a);
    case 1: return launch_dtype<_Float16>(a);
    default: return launch_dtype<__bf16>(a);
    }
}

}  // namespace fa
