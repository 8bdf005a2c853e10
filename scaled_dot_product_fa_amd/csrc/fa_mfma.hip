// fa_mfma.hip -- FlashAttention-2 forward for gfx950 on bf16/fp16 MFMA.
//
// Method (FlashAttention-2 forward article, wsisp.com: host wrapper, launch
// grid, fwd_flash_attn_kernel and _attn_fwd_inner; "Triton Ascend Attention",
// online softmax section): one workgroup per block of BM query rows of one
// (batch, head); K/V stream through LDS in tiles of BN keys; per query row a
// running max m, running sum l and an unnormalised fp32 accumulator are
// updated per tile with the rescale factor alpha = exp(m_old - m_new); the
// output is divided by l once at the end and m + log(l) is stored.  Causal
// tiles beyond the block's diagonal are never loaded, and only tiles that
// straddle the diagonal (or the ragged end of the keys) are masked, keeping
// key j for query i when j <= i ("flash-attention-kernel" skill page).
//
// gfx950 mapping (our design, not the article's):
//   * Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_{bf16,f16}: A = 32 keys x 16 dims from LDS,
//     B = 16 dims x 32 queries held in VGPRs for the whole kernel.  In the
//     32x32 accumulator every lane then owns one query column, so the row max
//     and row sum are in-lane reductions plus one exchange between the two
//     32-lane halves (v_permlane32_swap).
//   * The K rows feeding A are read in a permuted order (bits 2 and 3 of the
//     row index swapped) so that each lane's 16 accumulator values are 2 runs
//     of 8 consecutive keys.  The probabilities, rounded to the I/O type,
//     are then directly the B operand of O^T += V^T P^T (again
//     32x32x16), with no data movement between lanes.
//   * Three kernels share this mapping and differ in how K/V reach LDS and
//     how the work is overlapped:
//       - fa_fwd_mfma_kernel (pipe 0): K/V staged through VGPRs, V
//         transposed while it is stored (V^T, keys fastest) so the PV A
//         operand is one 16-byte read; two buffers, one barrier per tile;
//       - fa_fwd_mfma_dma_kernel (pipe 2): K/V loaded straight into LDS
//         (global_load_lds_dwordx4), V^T read with transposing LDS reads,
//         the QK^T of tile j+1 software-pipelined under the softmax of tile
//         j; its GEN instantiation serves strided views and the local window;
//       - fa_fwd_mfma_pp_kernel (pipe 3): the ping-pong kernel, in which the
//         two waves of each SIMD alternate MFMA and softmax phases (the
//         default for large grids; see its own comment).
//     The LDS tiles use XOR swizzles so the reads of a wave hit distinct
//     banks.
//   * exp2 is used with c = scale*log2(e) folded into one FMA per score:
//     p = exp2(s*c - m*c).  The stabiliser m only moves when the tile max
//     exceeds it by more than kLazyThreshold (log2 units), so the fp32
//     accumulator is rescaled rarely.  In exact arithmetic the softmax does
//     not depend on the stabiliser (l and the accumulator share it); in
//     finite precision it does unless l sums the same rounded p as the P.V
//     product (see Bf16Ops), which the bf16 kernels do.  p stays below
//     2^kLazyThreshold.
//   * Workgroup ids are remapped so one head's query blocks run on one XCD
//     (shared L2), and causal grids start with the longest blocks.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <string>
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// strided / windowed calls on large grids take the ping-pong kernel (1), or
// the software-pipelined kernel as on small grids (0)
#ifndef GENERAL_PP
#define GENERAL_PP 1
#endif
// key tile of the ping-pong kernel with a window at D = 128
#ifndef PP_WIN_BN
#define PP_WIN_BN 64
#endif
#ifndef PP_LEAD
#define PP_LEAD 4
#endif
#ifndef PP_PRIO
#define PP_PRIO 1
#endif


constexpr float kLog2e = 1.4426950408889634f;
// The running max is only raised when it grew by more than this many binary
// orders of magnitude; until then probabilities may reach 2^kLazyThreshold.
constexpr float kLazyThreshold = 8.0f;
// The ping-pong kernel instead keeps its stabiliser while every lane's
// partial row sum over a tile stays at or below this bound (2^15: any single
// p is then below the fp16 maximum of 65504).
constexpr float kPpSumBound = 32768.0f;
// A row that has not seen a key yet (m = -inf) forms its p against this
// stabiliser instead, -kPpUnseen: every key visible to it then gives
// p = +inf, its partial sums pass kPpSumBound and the max pass runs, so the
// first tile needs no test of its own; a tile that hides every key from it
// gives p = 0 and leaves it unseen.
constexpr float kPpUnseen = 3.0e38f;

// Normalisation in finite precision.  O's numerator sums the probabilities
// as rounded for the P.V product, so O is a convex combination of V rows
// only if its denominator sums those same rounded values.  A denominator of
// unrounded fp32 p leaves the rounding error of a dominant key (relative
// u = 2^-8 in bf16) in the numerator alone, a bias of up to u*|v| that comes
// on top of O's own rounding.  So bf16 kernels keep two row sums: the
// rounded one (summed with v_dot2 against 1.0, one op per packed pair)
// divides O, and the fp32 one gives the row statistic m + ln l, which the
// rounded sum would move by up to u on rows with few keys.  In fp16
// (u = 2^-11) the same bias is below 2^-11 * max|v|, so fp16 kernels divide
// by the fp32 sum.
struct Bf16Ops {
    static constexpr bool kRoundedNorm = true;
    static constexpr bool kSumRounded = false;
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two floats -> one dword, round to nearest even, first value low
    static __device__ __forceinline__ uint32_t pack2(float x, float y)
    {
        bf16x2 r = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, r);
    }
    // s + both values of a packed pair (as rounded)
    static __device__ __forceinline__ float add2(uint32_t x, float s)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                               __builtin_bit_cast(bf16x2, 0x3f803f80u), s,
                                               false);
    }
};

// fp16 I/O (ping-pong kernels): the row sum l, for O and for the LSE alike,
// is the sum of the rounded p (one v_dot2 per pair instead of an fp32 add per
// score).  It is then exactly the weight P.V used.  fp16 rows keep their
// stabiliser at the row max, so l >= 1 once a row has seen a key, and each
// rounded p is within 2^-11 of p (relative) or 2^-25 (absolute, subnormal):
// the sum moves by at most 2^-11 * l + Lk * 2^-25 <= 2^-10 * l for Lk <=
// 16384, and the LSE by at most 9.8e-4 in that worst case (every p rounded
// the same way).
struct F16Ops {
    static constexpr bool kRoundedNorm = false;
    static constexpr bool kSumRounded = true;
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y)
    {
        f16x2 r = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(uint32_t, r);
    }
    static __device__ __forceinline__ float add2(uint32_t x, float s)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x),
                                      __builtin_bit_cast(f16x2, 0x3c003c00u), s, false);
    }
};

// When the ping-pong kernel does move its stabiliser, bf16 rows place it this
// many binary orders above the row max, so that later, larger keys fit under
// the bound without another move.  bf16 has the exponent range: a p that is
// 24 + 100 orders below the max is still a normal number, and anything
// smaller is negligible.  fp16 would push small probabilities into its
// subnormals, so fp16 rows use the max itself.
template <typename Ops>
constexpr float pp_headroom()
{
    return std::is_same<Ops, Bf16Ops>::value ? 24.0f : 0.0f;
}

// Exchange between lane l and lane l ^ 32, combined with op.  With both
// operands equal, v_permlane32_swap leaves one copy of each half in each
// result, so op(r0, r1) is op(x[l % 32], x[l % 32 + 32]) in every lane.
__device__ __forceinline__ float half_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                              false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swap bits 2 and 3 of a row index within a 32-row key block.
__device__ __forceinline__ int swap_bits23(int r)
{
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int BH, Lq, Lk, ntq;
    float scale, c;  // c = scale * log2(e)
    // strided / windowed calls only (the GEN kernels): heads per batch,
    // element strides (batch, head, row) of q, k, v, o, window bounds (-1:
    // none)
    int H, wl, wr;
    int64_t qs[3], ks[3], vs[3], os[3];
};

// Workgroup id -> (head bh, query block qt).  Hardware places workgroup w
// on XCD w % 8; consecutive logical ids are made to share an XCD.
// `grouped` (causal calls with a left window edge): see below.
__device__ __forceinline__ void decompose(int wg, int nwg, int BH, int ntq,
                                          bool causal, int &bh, int &qt, bool grouped = false)
{
    const int per = nwg >> 3, rem = nwg & 7;
    const int xcd = wg & 7, idx = wg >> 3;
    if (causal && (BH & 7) == 0) {
        // each XCD owns BH/8 heads; longest query blocks first
        const int hpx = BH >> 3;
        // grouped: the heads g at a time (g: the fewest heads, dividing
        // BH/8, whose blocks fill the XCD's 32 CUs), longest blocks of the
        // group first, so that the blocks of few heads stream the same K/V
        // tiles together.  It gains where the window keeps the blocks'
        // work alike (+5% at 4096 rows with a 1024-key window) but loses a
        // little on plain causal calls, whose longest-first order over all
        // the XCD's heads balances better.
        int g = hpx;
        if (grouped) {
            g = 1;
            while (g < hpx && (g * ntq < 32 || hpx % g != 0)) ++g;
        }
        const int grp = idx / (g * ntq), r = idx % (g * ntq);
        qt = ntq - 1 - r / g;
        bh = xcd * hpx + grp * g + r % g;
        return;
    }
    const int logical = xcd < rem ? xcd * (per + 1) + idx
                                  : rem * (per + 1) + (xcd - rem) * per + idx;
    bh = logical / ntq;
    qt = logical % ntq;
    if (causal) qt = ntq - 1 - qt;
}

template <typename Ops, int D, bool CAUSAL, int NW, int QB, int BN, int OCC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_fwd_mfma_kernel(Params p)
{
    constexpr int NT = NW * 64;          // threads
    constexpr int BM = NW * QB * 32;     // query rows per workgroup
    constexpr int DC = D / 16;           // 16-dim chunks (k of the QK^T MFMA)
    constexpr int DB = D / 32;           // 32-dim blocks (rows of O^T)
    constexpr int KB = BN / 32;          // 32-key blocks (rows of S^T)
    constexpr int KC = BN / 16;          // 16-key chunks (k of the PV MFMA)
    constexpr int KROW = D * 2;          // bytes per K row in LDS
    constexpr int VROW = BN * 2;         // bytes per V^T row in LDS
    constexpr int KCH = D / 8;           // 16-byte chunks per K row
    constexpr int VCH = BN / 8;          // 16-byte chunks per V^T row
    constexpr int KBYTES = BN * KROW;
    constexpr int VBYTES = D * VROW;
    constexpr int BUF = KBYTES + VBYTES;
    constexpr int K_PER_T = BN * KCH / NT;       // K chunks loaded per thread
    constexpr int V_KEYS = BN * (D / 8) / NT;    // keys per thread in the V load
    static_assert(K_PER_T >= 1 && BN * KCH % NT == 0, "K tile split");
    static_assert(V_KEYS == 1 || V_KEYS == 2 || V_KEYS == 4 || V_KEYS == 8, "V tile split");
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    decompose(blockIdx.x, gridDim.x, p.BH, p.ntq, CAUSAL, bh, qt);
    const int q_first = qt * BM;
    const int qw = q_first + wave * QB * 32;  // first query row of this wave

    const uint16_t *qh = p.q + (int64_t)bh * p.Lq * D;
    const uint16_t *kh = p.k + (int64_t)bh * p.Lk * D;
    const uint16_t *vh = p.v + (int64_t)bh * p.Lk * D;

    // ---- Q^T operand, resident in VGPRs: lane holds 8 dims of its query.
    u32x4 qreg[QB][DC];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = qw + b * 32 + l32;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < p.Lq)
                x = *reinterpret_cast<const u32x4 *>(qh + (uint32_t)row * D + dc * 16 + hi * 8);
            qreg[b][dc] = x;
        }
    }

    f32x16 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][b][i] = 0.f;
    // l_part: fp32 row sum (for the row statistic); l_rnd: sum of the
    // rounded p (divides O; bf16 only, see Bf16Ops)
    float m_run[QB], l_part[QB], l_rnd[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        m_run[b] = -INFINITY;
        l_part[b] = 0.f;
        l_rnd[b] = 0.f;
    }

    const int kv_end = CAUSAL ? min(p.Lk, q_first + BM) : p.Lk;
    const int ntiles = (kv_end + BN - 1) / BN;

    // ---- global -> register staging of one K/V tile
    u32x4 kst[K_PER_T];
    u32x4 vst[V_KEYS];
    // V load split: thread owns V_KEYS consecutive keys x 8 dims
    const int v_dc = tid % (D / 8);
    const int v_kg = tid / (D / 8);

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int r = 0; r < K_PER_T; ++r) {
            const int ci = tid + NT * r;
            const int row = ci / KCH, c = ci % KCH;
            const int key = k0 + row;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < p.Lk)
                x = *reinterpret_cast<const u32x4 *>(kh + (uint32_t)key * D + c * 8);
            kst[r] = x;
        }
#pragma unroll
        for (int r = 0; r < V_KEYS; ++r) {
            const int key = k0 + v_kg * V_KEYS + r;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < p.Lk)
                x = *reinterpret_cast<const u32x4 *>(vh + (uint32_t)key * D + v_dc * 8);
            vst[r] = x;
        }
    };

    auto store_tile = [&](int buf) {
        uint8_t *kb = smem + buf * BUF;
        uint8_t *vb = kb + KBYTES;
#pragma unroll
        for (int r = 0; r < K_PER_T; ++r) {
            const int ci = tid + NT * r;
            const int row = ci / KCH, c = ci % KCH;
            const int pc = c ^ (swap_bits23(row & 15) & (KCH - 1));
            *reinterpret_cast<u32x4 *>(kb + row * KROW + pc * 16) = kst[r];
        }
        // transpose V_KEYS keys x 8 dims into 8 rows of V^T
        const int key0 = v_kg * V_KEYS;
        const int ch = key0 >> 3;            // 16-byte chunk within the V^T row
        const int off = (key0 & 7) * 2;      // byte offset within the chunk
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = v_dc * 8 + e;
            const int pc = ch ^ (((d >> 3) ^ d) & (VCH - 1));
            uint8_t *dst = vb + d * VROW + pc * 16 + off;
            if constexpr (V_KEYS == 1) {
                const uint32_t a = vst[0][e >> 1];
                *reinterpret_cast<uint16_t *>(dst) = (uint16_t)((e & 1) ? (a >> 16) : a);
                continue;
            }
            uint32_t w[V_KEYS / 2 > 0 ? V_KEYS / 2 : 1];
#pragma unroll
            for (int r = 0; r < V_KEYS / 2; ++r) {
                const uint32_t a = vst[2 * r][e >> 1];
                const uint32_t b = vst[2 * r + 1][e >> 1];
                w[r] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                               : ((a & 0xffffu) | (b << 16));
            }
            if constexpr (V_KEYS == 2) {
                *reinterpret_cast<uint32_t *>(dst) = w[0];
            } else if constexpr (V_KEYS == 4) {
                u32x2 x = {w[0], w[1]};
                *reinterpret_cast<u32x2 *>(dst) = x;
            } else {
                u32x4 x = {w[0], w[1], w[2], w[3]};
                *reinterpret_cast<u32x4 *>(dst) = x;
            }
        }
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    const float c = p.c;
    // K row this lane feeds into the A operand of S^T = K Q^T
    const int krow_lane = swap_bits23(l32);

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const int k0 = j * BN;
        const bool has_next = j + 1 < ntiles;
        if (has_next) load_tile(k0 + BN);

        const bool wave_idle = (qw >= p.Lq) || (CAUSAL && k0 > qw + QB * 32 - 1);
        if (!wave_idle) {
            const uint8_t *kb = smem + buf * BUF;
            const uint8_t *vb = kb + KBYTES;

            // ---- S^T = K Q^T (raw scores, fp32)
            f32x16 s[KB][QB];
#pragma unroll
            for (int kb_i = 0; kb_i < KB; ++kb_i)
#pragma unroll
                for (int b = 0; b < QB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kb_i][b][i] = 0.f;
#pragma unroll
            for (int kb_i = 0; kb_i < KB; ++kb_i) {
                const int row = kb_i * 32 + krow_lane;
                const int sw = swap_bits23(row & 15) & (KCH - 1);
#pragma unroll
                for (int dc = 0; dc < DC; ++dc) {
                    const int pc = (dc * 2 + hi) ^ sw;
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + row * KROW + pc * 16);
#pragma unroll
                    for (int b = 0; b < QB; ++b) s[kb_i][b] = Ops::mma(a, qreg[b][dc], s[kb_i][b]);
                }
            }

            // ---- masking: ragged key end, and the diagonal when causal
            const bool need_mask = (k0 + BN > p.Lk) || (CAUSAL && k0 + BN - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int kb_i = 0; kb_i < KB; ++kb_i)
#pragma unroll
                    for (int b = 0; b < QB; ++b)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = k0 + kb_i * 32 + (i >> 3) * 16 + hi * 8 + (i & 7);
                            const int qry = qw + b * 32 + l32;
                            const bool keep = key < p.Lk && (!CAUSAL || key <= qry);
                            s[kb_i][b][i] = keep ? s[kb_i][b][i] : -INFINITY;
                        }
            }

            // ---- online softmax per query block; P^T packed for the B operand
            u32x4 pk[KC][QB];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb_i = 0; kb_i < KB; ++kb_i)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb_i][b][i]);
                mx = half_max(mx);
                const float m_new = fmaxf(m_run[b], mx);
                const bool grow = (m_new - m_run[b]) * c > kLazyThreshold;
                if (__any(grow)) {
                    // m_run = -inf gives alpha = 0 (nothing accumulated yet)
                    const float alpha = (m_new == -INFINITY)
                                            ? 1.f
                                            : __builtin_amdgcn_exp2f((m_run[b] - m_new) * c);
                    m_run[b] = m_new;
                    l_part[b] *= alpha;
                    if constexpr (Ops::kRoundedNorm) l_rnd[b] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][b][i] *= alpha;
                }
                const float mc = (m_run[b] == -INFINITY) ? 0.f : m_run[b] * c;
                float rs = 0.f, rr = 0.f;
#pragma unroll
                for (int kb_i = 0; kb_i < KB; ++kb_i) {
                    float e[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        e[i] = __builtin_amdgcn_exp2f(fmaf(s[kb_i][b][i], c, -mc));
                        rs += e[i];
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        u32x4 x;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            x[w] = Ops::pack2(e[h * 8 + 2 * w], e[h * 8 + 2 * w + 1]);
                            if constexpr (Ops::kRoundedNorm) rr = Ops::add2(x[w], rr);
                        }
                        pk[kb_i * 2 + h][b] = x;
                    }
                }
                l_part[b] += rs;
                if constexpr (Ops::kRoundedNorm) l_rnd[b] += rr;
            }

            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + l32;
                const int sw = ((d >> 3) ^ d) & (VCH - 1);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int pc = (kc * 2 + hi) ^ sw;
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(vb + d * VROW + pc * 16);
#pragma unroll
                    for (int b = 0; b < QB; ++b) oacc[db][b] = Ops::mma(a, pk[kc][b], oacc[db][b]);
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, rounded to nearest even; LSE = m*scale + ln l
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float l = half_sum(l_part[b]);
        const float ln = Ops::kRoundedNorm ? half_sum(l_rnd[b]) : l;
        const int row = qw + b * 32 + l32;
        if (row < p.Lq) {
            const float inv = ln > 0.f ? 1.f / ln : 0.f;
            uint16_t *orow = p.o + ((int64_t)bh * p.Lq + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + g * 8 + hi * 4;
                    u32x2 x = {Ops::pack2(oacc[db][b][4 * g] * inv, oacc[db][b][4 * g + 1] * inv),
                               Ops::pack2(oacc[db][b][4 * g + 2] * inv, oacc[db][b][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(orow + d) = x;
                }
            if (p.lse != nullptr && hi == 0)
                p.lse[(int64_t)bh * p.Lq + row] =
                    l > 0.f ? m_run[b] * p.scale + __logf(l) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Direct-load variant.  K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at the wave's
// LDS base + 16*i), so no VGPRs hold staged data and no LDS stores are
// issued.  Both tiles stay row-major (key rows of D elements) with 16-byte
// chunks XOR-swizzled by row; the swizzle is applied by choosing which global
// chunk each lane fetches.  The V^T operand of the PV product is read with
// ds_read_b64_tr_b16, which transposes 16-bit data inside each 16-lane group:
// lane t receives element t%4 of the 8-byte blocks addressed by lanes
// 4r + t/4 (r = 0..3).  So the lanes of a group address a 4-key x 16-dim
// block and each lane gets 4 consecutive keys of one dim.  Two such reads
// give the 8 keys of one lane's A operand.
// ---------------------------------------------------------------------------

// LDS swizzles for 64 banks of 4 bytes (256 bytes per bank cycle).
//
// K: a 16-byte read phase serves 16 lanes, which fetch rows
// swap_bits23(0..15) of a 32-row block at one logical chunk.  D = 128 rows
// are 256 bytes (every row starts on bank 0): XOR with the same permutation
// gives the 16 lanes 16 distinct chunks.  D = 64 rows are 128 bytes (row
// parity picks the bank half): XOR with the permutation shifted down by one
// gives each parity class 8 distinct chunks.
template <int D>
__device__ __forceinline__ int swz_k(int row)
{
    if constexpr (D == 128) return swap_bits23(row & 15);
    return (swap_bits23(row & 15) >> 1) & 7;
}

// V: an 8-byte transposed read phase serves 32 lanes, which touch 4
// consecutive rows x 4 adjacent chunks (16 x 16 bytes).  D = 128: XOR the
// chunk with 4*(row % 4) so each row lands on its own 64-byte bank quarter.
// D = 64: rows r and r+2 share a bank half, so XOR with 4*((row/2) % 2).
template <int D>
__device__ __forceinline__ int swz_v(int row)
{
    if constexpr (D == 128) return 4 * (row & 3);
    return 4 * ((row >> 1) & 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ uint2 ds_read_tr(const uint8_t *p)
{
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

// The same read at an LDS byte address.
__device__ __forceinline__ uint2 ds_read_tr_at(uint32_t a)
{
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)a);
    return __builtin_bit_cast(uint2, r);
}

// One global_load_lds_dwordx4: the wave's 64 lanes each fetch 16 bytes from
// their own global address and the hardware writes them to LDS at m0 +
// 16 * lane.  Issued from inline assembly on purpose: the compiler treats
// its own LDS-DMA instruction as a FLAT access that may target LDS, and while
// one is in flight it then waits for every outstanding LDS read (lgkmcnt(0))
// before each use of any of them, which exposes the full LDS latency on every
// MFMA operand.  Hidden from the compiler, the DMA only counts against
// vmcnt, and the kernel orders it with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma_16B(const void *src, uint32_t lds_dst)
{
    __asm__ volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

// The same load with a wave-uniform 64-bit base (SGPRs) and a per-lane
// 32-bit byte offset.  No memory clobber: the loads target LDS buffers that
// no wave reads before the next barrier, so LDS reads may move across them.
__device__ __forceinline__ void dma_16B_sbase(const void *base, uint32_t off, uint32_t lds_dst)
{
    __asm__ volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_dst));
}

// LDS byte address of a __shared__ object (for m0).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// A 16-byte LDS load (ds_read_b128) from an LDS byte address.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ u32x4 lds_load_b128(uint32_t a)
{
    return *(const lds_u32x4 *)(uintptr_t)a;
}

// An LDS store the compiler does not see as a memory access.  A tile loop
// that holds an LDS store the compiler knows of, even on a rare path and
// even as asm behind a memory clobber, loses the read-ahead schedule of its
// MFMA phases; a rare path that stages data through LDS stores with this.
// The compiler orders a later read after it only through data: the store
// takes the base address `base` of the staged data as an in-out operand,
// so every address formed from the returned base follows the store (and a
// wave's LDS operations complete in issue order).
__device__ __forceinline__ void ds_store_b64_opaque(uint32_t &base, uint32_t off, u32x2 v)
{
    __asm__ volatile("ds_write_b64 %1, %2" : "+v"(base) : "v"(base + off), "v"(v));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// GEN: strided views and the local window (runtime strides in Params, key
// range clipped to the window, window edges masked); otherwise contiguous
// [B, H, L, D] with compile-time row strides.
template <typename Ops, int D, bool CAUSAL, int NW, int QB, int BN, int OCC, bool GEN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_fwd_mfma_dma_kernel(Params p)
{
    constexpr int NT = NW * 64;
    constexpr int BM = NW * QB * 32;     // query rows per workgroup
    constexpr int DC = D / 16;           // 16-dim chunks (k of the QK^T MFMA)
    constexpr int DB = D / 32;           // 32-dim blocks (rows of O^T)
    constexpr int KB = BN / 32;          // 32-key blocks (rows of S^T)
    constexpr int KC = BN / 16;          // 16-key chunks (k of the PV MFMA)
    constexpr int ROWB = D * 2;          // bytes per K or V row in LDS
    constexpr int KCH = D / 8;           // 16-byte chunks per row
    constexpr int TILEB = BN * ROWB;     // bytes of one K (or V) tile
    constexpr int LOADS = TILEB / (NT * 16);
    constexpr int NQK = KB * DC;         // K reads (A operands) per QK^T
    constexpr int HALF = NQK / 2;        // ... issued before the rescale branch
    static_assert(LOADS >= 1 && TILEB % (NT * 16) == 0, "tile split");
    static_assert(BN % 32 == 0 && D % 32 == 0 && KC >= 2, "tile shape");

    // Two buffers per operand (separate objects; the DMA into one overlaps
    // the reads of the other).
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar, so LDS DMA destinations stay in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    decompose(blockIdx.x, gridDim.x, p.BH, p.ntq, CAUSAL, bh, qt);
    const int q_first = qt * BM;
    const int qw = q_first + wave * QB * 32;   // first query row of this wave

    // per-(b, h) bases and row strides, in elements
    int64_t q_base, k_base, v_base, o_base;
    int q_sl, k_sl, v_sl, o_sl;
    if constexpr (GEN) {
        const int b = bh / p.H, h = bh % p.H;
        q_base = b * p.qs[0] + h * p.qs[1];
        k_base = b * p.ks[0] + h * p.ks[1];
        v_base = b * p.vs[0] + h * p.vs[1];
        o_base = b * p.os[0] + h * p.os[1];
        q_sl = (int)p.qs[2];
        k_sl = (int)p.ks[2];
        v_sl = (int)p.vs[2];
        o_sl = (int)p.os[2];
    } else {
        q_base = (int64_t)bh * p.Lq * D;
        k_base = (int64_t)bh * p.Lk * D;
        v_base = k_base;
        o_base = q_base;
        q_sl = k_sl = v_sl = o_sl = D;
    }
    const uint16_t *qh = p.q + q_base;
    const uint16_t *kh = p.k + k_base;
    const uint16_t *vh = p.v + v_base;

    // ---- Q^T operand in VGPRs (rows past Lq read the last row; not stored)
    u32x4 qreg[QB][DC];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = min(qw + b * 32 + l32, p.Lq - 1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            qreg[b][dc] = *reinterpret_cast<const u32x4 *>(qh + (int64_t)row * q_sl + dc * 16 + hi * 8);
    }

    // ---- per-lane DMA source offsets (bytes within a tile) and LDS slots
    int ld_row[LOADS];
    uint32_t ld_k[LOADS], ld_v[LOADS];
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
        const int slot = (r * NW + wave) * 64 + lane;
        const int row = slot / KCH, pc = slot % KCH;
        ld_row[r] = row;
        ld_k[r] = (uint32_t)(row * k_sl + (pc ^ swz_k<D>(row)) * 8) * 2;
        ld_v[r] = (uint32_t)(row * v_sl + (pc ^ swz_v<D>(row)) * 8) * 2;
    }
    auto issue_one = [&](const uint16_t *src, const uint32_t *offs, int sl, int k0, uint8_t *dst) {
        const uint8_t *t = reinterpret_cast<const uint8_t *>(src + (int64_t)k0 * sl);
        // wave-uniform LDS base of this wave's 1 KB slots (an SGPR)
        const uint32_t dbase = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(lds_addr(dst) + (uint32_t)(wave * 1024)));
        if (k0 + BN <= p.Lk) {   // uniform: every row of the tile exists
#pragma unroll
            for (int r = 0; r < LOADS; ++r)
                dma_16B(t + offs[r], dbase + (uint32_t)(r * NW * 1024));
            return;
        }
        const int last = p.Lk - 1 - k0;  // last valid row of this tile
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            uint32_t o = offs[r];
            if (ld_row[r] > last) {
                // past the end of the keys: fetch any valid row (its scores
                // are masked and its V rows get probability 0)
                o -= (uint32_t)(ld_row[r] - last) * (uint32_t)(sl * 2);
            }
            dma_16B(t + o, dbase + (uint32_t)(r * NW * 1024));
        }
    };
    auto issue_k = [&](int k0, uint8_t *kd) { issue_one(kh, ld_k, k_sl, k0, kd); };
    auto issue_v = [&](int k0, uint8_t *vd) { issue_one(vh, ld_v, v_sl, k0, vd); };

    // ---- per-lane LDS read offsets (loop invariant)
    uint32_t k_rd[DC];
    {
        const int row = swap_bits23(l32);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            k_rd[dc] = (uint32_t)(row * ROWB + (((dc * 2 + hi) ^ swz_k<D>(row)) * 16));
    }
    uint32_t v_rd[DB];
    {
        const int g = lane >> 4, t = lane & 15;
        const int row = 8 * hi + (t >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (g & 1) + 4 * (t & 3);   // element
            const int c = col >> 3, within = (col & 7) * 2;
            v_rd[db] = (uint32_t)(row * ROWB + ((c ^ swz_v<D>(row)) * 16) + within);
        }
    }

    f32x16 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][b][i] = 0.f;
    // l_part: fp32 row sum (for the row statistic); l_rnd: sum of the
    // rounded p (divides O; bf16 only, see Bf16Ops)
    float m_run[QB], l_part[QB], l_rnd[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        m_run[b] = -INFINITY;
        l_part[b] = 0.f;
        l_rnd[b] = 0.f;
    }
    const float c = p.c;

    // keys [kv_begin, kv_end) are visible to some row of the block
    int kv_begin = 0;
    int kv_end = CAUSAL ? min(p.Lk, q_first + BM) : p.Lk;
    if constexpr (GEN) {
        if (p.wl >= 0) kv_begin = max(0, q_first - p.wl) / BN * BN;
        if (p.wr >= 0) kv_end = min(kv_end, q_first + BM + p.wr);
    }
    const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + BN - 1) / BN : 0;
    // a block that sees no key still runs the (unused) prologue loads: keep
    // them on tile 0, so that every issued tile starts below Lk
    if (ntiles == 0) kv_begin = 0;

    struct STile {
        f32x16 v[KB][QB];
    };
    // MFMAs n in [n0, n1) of S^T = K Q^T for one tile, ordered dc-major so
    // the KB*QB accumulators form independent chains; each K read (A
    // operand) feeds QB MFMAs.
    auto qk_part = [&](STile &st, const uint8_t *kbuf, int n0, int n1) {
#pragma unroll
        for (int n = n0; n < n1; ++n) {
            const int dc = n / KB, kb = n % KB;
            if (dc == 0) {
#pragma unroll
                for (int b = 0; b < QB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) st.v[kb][b][i] = 0.f;
            }
            const u32x4 a = *reinterpret_cast<const u32x4 *>(kbuf + k_rd[dc] + kb * 32 * ROWB);
#pragma unroll
            for (int b = 0; b < QB; ++b) st.v[kb][b] = Ops::mma(a, qreg[b][dc], st.v[kb][b]);
        }
    };
    auto sync_tiles = [&]() {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // Software pipeline: step j runs the QK^T MFMAs of tile j+1 while the
    // vector ALUs run the softmax of tile j, then adds P_j V_j.  K therefore
    // runs one tile ahead of V: during step j the DMA fills K_{j+2} and
    // V_{j+1}, into the buffers that K_j and V_{j-1} left at the end of step
    // j-1.  Each step is branch-free apart from the DMA guards and the mask at
    // its start and the rare rescale, and sched_group_barrier pins the MFMA /
    // LDS-read / VALU interleave of the two straight-line blocks.  Tiles past
    // a wave's diagonal are not skipped: they are fully masked and contribute
    // p = 0.
    issue_k(kv_begin, k_lds0);
    issue_v(kv_begin, v_lds0);
    if (ntiles > 1) issue_k(kv_begin + BN, k_lds1);
    sync_tiles();
    STile cur;
    qk_part(cur, k_lds0, 0, NQK);
    __syncthreads();   // everyone is done with K_0 before K_2 lands there

    // VALU slots per MFMA: one 8-key chunk of P costs 8 FMA + 8 exp + 8 add
    // + 4 convert; chunks 0-1 go under the second half of QK^T, chunks
    // 2..KC-1 under the PV MFMAs
    constexpr int VALU_P = 28;
    constexpr int VALU_B = (2 * VALU_P + HALF - 1) / HALF;
    constexpr int VALU_C = ((KC - 2) * VALU_P + 4 + DB * KC - 1) / (DB * KC);

    auto step = [&](int j, const uint8_t *k_next, const uint8_t *v_cur, uint8_t *k_dma,
                    uint8_t *v_dma) {
        if (j + 2 < ntiles) issue_k(kv_begin + (j + 2) * BN, k_dma);
        if (j + 1 < ntiles) issue_v(kv_begin + (j + 1) * BN, v_dma);
        const int k0 = kv_begin + j * BN;
        bool need_mask = (k0 + BN > p.Lk) || (CAUSAL && k0 + BN - 1 > qw);
        if constexpr (GEN)
            need_mask = need_mask || (p.wr >= 0 && k0 + BN - 1 > qw + p.wr) ||
                        (p.wl >= 0 && k0 < qw + QB * 32 - 1 - p.wl);
        if (need_mask) {
            // element i of block kb holds key k0 + hi*8 + c, c = kb*32 +
            // (i>>3)*16 + (i&7) a constant: kept when lo <= c <= top, with
            // the bounds folded per lane and row block (one compare each)
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int qrow = qw + b * 32 + l32;
                int top = p.Lk - 1 - k0;
                if (CAUSAL) top = min(top, qrow - k0);
                int lo = 0;
                if constexpr (GEN) {
                    if (p.wr >= 0) top = min(top, qrow + p.wr - k0);
                    if (p.wl >= 0) lo = qrow - p.wl - k0 - hi * 8;
                }
                top -= hi * 8;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int c = kb * 32 + (i >> 3) * 16 + (i & 7);
                        bool keep = c <= top;
                        if constexpr (GEN) keep = keep && c >= lo;
                        cur.v[kb][b][i] = keep ? cur.v[kb][b][i] : -INFINITY;
                    }
            }
        }
        // block A: row maxima of tile j | first half of QK^T for tile j+1
        STile nxt;
        float mx[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            // four independent partial maxima keep the chains short
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) m4[i & 3] = fmaxf(m4[i & 3], cur.v[kb][b][i]);
            mx[b] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        }
        qk_part(nxt, k_next, 0, HALF);
        float m_new[QB];
        bool grow = false;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            m_new[b] = fmaxf(m_run[b], half_max(mx[b]));
            grow = grow || (m_new[b] - m_run[b]) * c > kLazyThreshold;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // LDS read
#pragma unroll
        for (int n = 0; n < HALF; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);       // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, 2 * QB, 0);   // VALU
        }
        if (__any(grow)) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                // m_run = -inf gives alpha = 0 (nothing accumulated yet)
                const float alpha = (m_new[b] == -INFINITY)
                                        ? 1.f
                                        : __builtin_amdgcn_exp2f((m_run[b] - m_new[b]) * c);
                m_run[b] = m_new[b];
                l_part[b] *= alpha;
                if constexpr (Ops::kRoundedNorm) l_rnd[b] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][b][i] *= alpha;
            }
        }
        // block B: second half of QK^T for tile j+1 under the exponentials of
        // key chunks 0-1 of tile j; then O^T += V^T P^T chunk by chunk, with
        // the exponentials of the later chunks under the PV MFMAs of the
        // earlier ones.  That keeps MFMA and VALU work balanced inside each
        // phase.
        float mc[QB], r4[QB][4], rr[QB][2];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            mc[b] = (m_run[b] == -INFINITY) ? 0.f : m_run[b] * c;
#pragma unroll
            for (int w = 0; w < 4; ++w) r4[b][w] = 0.f;
            rr[b][0] = rr[b][1] = 0.f;
        }
        auto make_p = [&](int kc, int b) {
            const int kb = kc >> 1, h = kc & 1;
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = __builtin_amdgcn_exp2f(fmaf(cur.v[kb][b][h * 8 + i], c, -mc[b]));
                r4[b][i & 3] += e[i];
            }
            u32x4 x;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[w] = Ops::pack2(e[2 * w], e[2 * w + 1]);
                if constexpr (Ops::kRoundedNorm) rr[b][w & 1] = Ops::add2(x[w], rr[b][w & 1]);
            }
            return x;
        };
        u32x4 pk[KC][QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            pk[0][b] = make_p(0, b);
            pk[1][b] = make_p(1, b);
        }
        qk_part(nxt, k_next, HALF, NQK);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if (kc + 2 < KC) {
#pragma unroll
                for (int b = 0; b < QB; ++b) pk[kc + 2][b] = make_p(kc + 2, b);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint8_t *vp = v_cur + v_rd[db] + kc * 16 * ROWB;
                const uint2 lo = ds_read_tr(vp);
                const uint2 hi4 = ds_read_tr(vp + 4 * ROWB);
                const u32x4 a = {lo.x, lo.y, hi4.x, hi4.y};
#pragma unroll
                for (int b = 0; b < QB; ++b) oacc[db][b] = Ops::mma(a, pk[kc][b], oacc[db][b]);
            }
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            l_part[b] += (r4[b][0] + r4[b][1]) + (r4[b][2] + r4[b][3]);
            if constexpr (Ops::kRoundedNorm) l_rnd[b] += rr[b][0] + rr[b][1];
        }
        // K reads two MFMA groups ahead; the transposed V reads stay ahead of
        // the PV MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);                 // LDS read
#pragma unroll
        for (int n = HALF; n < NQK; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);            // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);             // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_B * QB, 1);   // VALU
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);                 // LDS read
#pragma unroll
        for (int n = 0; n < DB * KC; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);            // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);             // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_C * QB, 1);   // VALU
        }
        cur = nxt;
        sync_tiles();
    };
    for (int j = 0; j < ntiles; j += 2) {
        step(j, k_lds1, v_lds0, k_lds0, v_lds1);
        if (j + 1 >= ntiles) break;
        step(j + 1, k_lds0, v_lds1, k_lds1, v_lds0);
    }

    // ---- epilogue: O = acc / l, rounded to nearest even; LSE = m*scale + ln l
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float l = half_sum(l_part[b]);
        const float ln = Ops::kRoundedNorm ? half_sum(l_rnd[b]) : l;
        const int row = qw + b * 32 + l32;
        if (row < p.Lq) {
            const float inv = ln > 0.f ? 1.f / ln : 0.f;
            uint16_t *orow = p.o + o_base + (int64_t)row * o_sl;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + g * 8 + hi * 4;
                    u32x2 x = {Ops::pack2(oacc[db][b][4 * g] * inv, oacc[db][b][4 * g + 1] * inv),
                               Ops::pack2(oacc[db][b][4 * g + 2] * inv, oacc[db][b][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(orow + d) = x;
                }
            if (p.lse != nullptr && hi == 0)
                p.lse[(int64_t)bh * p.Lq + row] =
                    l > 0.f ? m_run[b] * p.scale + __logf(l) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Ping-pong variant (8 waves, 32 query rows each, BN-key tiles).  The two
// waves that share a SIMD (w and w + 4) run half a step apart: while one
// issues the MFMAs of its step (P_j V_j for tile j and S_{j+1} = Q K_{j+1}^T
// for the next tile, reading K and V from LDS), the other runs the softmax
// of its next tile on the vector ALU, and a workgroup barrier after every
// phase keeps the two groups in this alternation.  One "slot" is the time
// between two barriers; group 0 (waves 0-3) runs its MFMA phases in even
// slots and group 1 (waves 4-7) in odd slots:
//   group 0: QK_0 | SM_0 | PV_0+QK_1 | SM_1 | PV_1+QK_2 | ...
//   group 1:  --  | QK_0 | SM_0      | PV_0+QK_1 | SM_1 | ...
// so K_t is read in slots 2t and 2t+1 and V_t in slots 2t+2 and 2t+3.
// Every slot loads one tile, in pieces spread through both phases so that
// no wave stalls behind a burst of loads: slot 2s loads V_{s+1} and slot
// 2s+1 loads K_{s+2}, three LDS buffers each.  Before each barrier a wave
// waits for its loads of all earlier slots (vmcnt), so every load has more
// than a slot to land.  (Reading the first V operands of an MFMA phase
// already in the softmax phase before it, which the early visibility
// allows, measured slower: those reads compete with the partner's MFMA
// phase.)
// ---------------------------------------------------------------------------
// GEN: strided views (runtime strides); WIN: the local window (with GEN).
template <typename Ops, int D, bool CAUSAL, int BN, bool GEN = false, bool WIN = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_mfma_pp_kernel(Params p)
{
    constexpr int NW = 8;
    constexpr int BM = NW * 32;          // query rows per workgroup
    constexpr int DC = D / 16;           // 16-dim chunks (k of the QK^T MFMA)
    constexpr int DB = D / 32;           // 32-dim blocks (rows of O^T)
    constexpr int KB = BN / 32;          // 32-key blocks (rows of S^T)
    constexpr int KC = BN / 16;          // 16-key chunks (k of the PV MFMA)
    constexpr int ROWB = D * 2;          // bytes per K or V row in LDS
    constexpr int KCH = D / 8;           // 16-byte chunks per row
    constexpr int TILEB = BN * ROWB;     // bytes of one K (or V) tile
    constexpr int LOADS = TILEB / (NW * 64 * 16);   // loads per wave per tile
    static_assert(LOADS >= 1 && TILEB % (NW * 64 * 16) == 0, "tile split");
    static_assert(6 * TILEB <= 160 * 1024, "three K and three V buffers fit the LDS");

    __shared__ __attribute__((aligned(1024))) uint8_t k_lds[3][TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds[3][TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;           // waves w and w+4 share a SIMD
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    decompose(blockIdx.x, gridDim.x, p.BH, p.ntq, CAUSAL, bh, qt, WIN && p.wl >= 0);
    const int q_first = qt * BM;
    const int qw = q_first + wave * 32;   // first query row of this wave
    const int qrow = qw + l32;            // this lane's query row

    // per-(b, h) bases and row strides, in elements (GEN: strided views)
    int64_t qg_base, kg_base, vg_base, og_base;
    int q_sl, k_sl, v_sl, o_sl;
    if constexpr (GEN) {
        const int b = bh / p.H, h = bh % p.H;
        qg_base = b * p.qs[0] + h * p.qs[1];
        kg_base = b * p.ks[0] + h * p.ks[1];
        vg_base = b * p.vs[0] + h * p.vs[1];
        og_base = b * p.os[0] + h * p.os[1];
        q_sl = (int)p.qs[2];
        k_sl = (int)p.ks[2];
        v_sl = (int)p.vs[2];
        o_sl = (int)p.os[2];
    } else {
        qg_base = (int64_t)bh * p.Lq * D;
        kg_base = (int64_t)bh * p.Lk * D;
        vg_base = kg_base;
        og_base = qg_base;
        q_sl = k_sl = v_sl = o_sl = D;
    }
    const uint16_t *qh = p.q + qg_base;
    const uint16_t *kh = p.k + kg_base;
    const uint16_t *vh = p.v + vg_base;

    // ---- Q^T operand in VGPRs (rows past Lq read the last row; not stored)
    u32x4 qreg[DC];
    {
        const int row = min(qrow, p.Lq - 1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            qreg[dc] = *reinterpret_cast<const u32x4 *>(
                qh + (GEN ? (int64_t)row * q_sl : (int64_t)((uint32_t)row * D)) + dc * 16 + hi * 8);
    }

    // keys [kv_begin, kv_end) are visible to some row of the block (WIN:
    // clipped to the window)
    int kv_begin = 0;
    int kv_end = CAUSAL ? min(p.Lk, q_first + BM) : p.Lk;
    if constexpr (WIN) {
        if (p.wl >= 0) kv_begin = max(0, q_first - p.wl) / BN * BN;
        if (p.wr >= 0) kv_end = min(kv_end, q_first + BM + p.wr);
    }
    const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + BN - 1) / BN : 0;

    // ---- loads: per-lane source offsets (bytes within a tile).
    // A wave's softmax phases always load one tensor and its MFMA phases the
    // other (group 0: K in softmax phases, V in MFMA phases; group 1 the
    // reverse), so the whole-tile offsets of both kinds are fixed per wave.
    int ld_row[LOADS];
    uint32_t ld_sm[LOADS], ld_mf[LOADS];
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
        const int slot = (r * NW + wave) * 64 + lane;
        const int row = slot / KCH, pc = slot % KCH;
        ld_row[r] = row;
        const uint32_t ov = (uint32_t)(row * v_sl + (pc ^ swz_v<D>(row)) * 8) * 2;
        const uint32_t ok = (uint32_t)(row * k_sl + (pc ^ swz_k<D>(row)) * 8) * 2;
        ld_sm[r] = grp == 0 ? ok : ov;
        ld_mf[r] = grp == 0 ? ov : ok;
    }
    const uint32_t k_base = lds_addr(k_lds[0]), v_base = lds_addr(v_lds[0]);
    // The loads of one phase, worked out before its straight-line block: the
    // tile's global base, the LDS destination of this wave's first piece and
    // the per-lane byte offsets (`whole`: those of a tile that lies entirely
    // below Lk).  Tile t goes to buffer t % 3.  Past the last tile the last
    // tile is fetched again (into the buffer of the requested tile, which no
    // wave reads any more), so every slot issues the same loads; rows past
    // the end of the keys fetch the last valid row (their scores are masked
    // and their V rows get probability 0).  Only a ragged tile pays for the
    // per-lane clamp.
    struct LoadPlan {
        const uint16_t *src;
        uint32_t dst;
        uint32_t off[LOADS];
    };
    auto plan = [&](bool is_k, int tile, const uint32_t (&whole)[LOADS]) {
        LoadPlan pl;
        const int k0 = kv_begin + min(tile, ntiles - 1) * BN;
        const int sl = is_k ? k_sl : v_sl;
        pl.src = (is_k ? kh : vh) + (int64_t)k0 * sl;
        pl.dst = (is_k ? k_base : v_base) + (uint32_t)((tile % 3) * TILEB) +
                 (uint32_t)(wave * 1024);
        const int last = p.Lk - 1 - k0;
#pragma unroll
        for (int r = 0; r < LOADS; ++r) pl.off[r] = whole[r];
        if (last < BN - 1) {
#pragma unroll
            for (int r = 0; r < LOADS; ++r)
                pl.off[r] -= (uint32_t)max(ld_row[r] - last, 0) * (uint32_t)sl * 2u;
        }
        return pl;
    };
    // the prologue's loads, of either tensor
    auto plan_kv = [&](bool is_k, int tile) {
        return plan(is_k, tile, (grp == 0) == is_k ? ld_sm : ld_mf);
    };
    auto issue = [&](const LoadPlan &pl, int r) {
        dma_16B_sbase(pl.src, pl.off[r], pl.dst + (uint32_t)(r * NW * 1024));
    };

    // ---- per-lane LDS read offsets (loop invariant)
    uint32_t k_rd[DC];
    {
        const int row = swap_bits23(l32);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            k_rd[dc] = (uint32_t)(row * ROWB + (((dc * 2 + hi) ^ swz_k<D>(row)) * 16));
    }
    uint32_t v_rd[DB];
    {
        const int g = lane >> 4, t = lane & 15;
        const int row = 8 * hi + (t >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (g & 1) + 4 * (t & 3);   // element
            const int c = col >> 3, within = (col & 7) * 2;
            v_rd[db] = (uint32_t)(row * ROWB + ((c ^ swz_v<D>(row)) * 16) + within);
            // opaque to the compiler: with the value's known zero bits it
            // would form every buffer's address with a fresh OR instead of
            // the read's offset field
            __asm__ volatile("" : "+v"(v_rd[db]));
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    // l_part: fp32 row sum (for the row statistic); l_rnd: sum of the
    // rounded p (divides O; bf16 only, see Bf16Ops)
    float m_run = -INFINITY, l_part = 0.f, l_rnd = 0.f;
    const float c = p.c;
    const float head = pp_headroom<Ops>() / c;   // in score units (c > 0 here)

    f32x16 st[KB];    // S^T of the tile whose softmax runs next
    u32x4 pk[KC];     // P^T (I/O type) of the tile whose PV runs next

    // S^T = K Q^T for one tile: A = 32 keys x 16 dims of K (LDS), B = Q^T.
    auto qk_mma = [&](const uint8_t *kbuf, int dc, int kb) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(kbuf + k_rd[dc] + kb * 32 * ROWB);
        if (dc == 0) {
            f32x16 z;
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = 0.f;
            st[kb] = Ops::mma(a, qreg[0], z);
        } else {
            st[kb] = Ops::mma(a, qreg[dc], st[kb]);
        }
    };
    // One MFMA phase: O^T += V^T P^T for tile j (A = 32 dims x 16 keys of V
    // from two transposed LDS reads, B = P^T), then S^T = K Q^T for tile j+1.
    // The last tile's phase also runs the QK^T half, on whatever the K
    // buffer holds (the result is never used), so that every phase is one
    // straight-line block.  The LDS reads are pinned PP_LEAD MFMAs ahead of
    // their use; the slot's loads are spread over the phase.
    constexpr int NPV = KC * DB, NQK = DC * KB;
    auto read_v = [&](const uint8_t *vbuf, int kc, int db) {
        const uint8_t *vp = vbuf + v_rd[db] + kc * 16 * ROWB;
        const uint2 lo = ds_read_tr(vp);
        const uint2 hi4 = ds_read_tr(vp + 4 * ROWB);
        return u32x4{lo.x, lo.y, hi4.x, hi4.y};
    };
    // the MFMA (PV first, then QK^T) after which load piece r is issued
    auto load_at = [](int r) { return 2 + r * ((NPV + NQK) / LOADS); };
    auto mfma_phase = [&](const LoadPlan &pl, const uint8_t *vbuf, const uint8_t *kbuf) {
        if (PP_PRIO) __builtin_amdgcn_s_setprio(PP_PRIO);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 a = read_v(vbuf, kc, db);
                oacc[db] = Ops::mma(a, pk[kc], oacc[db]);
#pragma unroll
                for (int r = 0; r < LOADS; ++r)
                    if (kc * DB + db == load_at(r)) issue(pl, r);
            }
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                qk_mma(kbuf, dc, kb);
#pragma unroll
                for (int r = 0; r < LOADS; ++r)
                    if (NPV + dc * KB + kb == load_at(r)) issue(pl, r);
            }
        constexpr int LEAD = PP_LEAD;
        constexpr int NM = NPV + NQK;
        static_assert(LEAD >= 1 && LEAD <= NPV, "read lead");
        // MFMA n (n < NPV: PV, else QK) is preceded by the reads of MFMA
        // n + LEAD
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
#pragma unroll
        for (int n = 0; n < NPV - LEAD; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int n = NPV - LEAD; n < NM - LEAD; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
        if (PP_PRIO) __builtin_amdgcn_s_setprio(0);
        // S must exist before the barrier
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" : "+v"(st[kb]));
    };
    // Online softmax of tile j in slot t (vector ALU only): mask, row max,
    // lazy rescale, p = exp2(s*c - m*c) rounded to the I/O type, row sum.
    auto softmax = [&](const LoadPlan &pl, int j) {
        const int k0 = kv_begin + j * BN;
        bool need_mask = (k0 + BN > p.Lk) || (CAUSAL && k0 + BN - 1 > qw);
        if constexpr (WIN)
            need_mask = need_mask || (p.wr >= 0 && k0 + BN - 1 > qw + p.wr) ||
                        (p.wl >= 0 && k0 < qw + 31 - p.wl);
        if (need_mask) {
            // element i of block kb holds key k0 + hi*8 + c with the constant
            // c = kb*32 + (i>>3)*16 + (i&7): kept when lo <= c <= top, the
            // per-lane bounds folded once (one compare per element)
            int top = p.Lk - 1 - k0;
            if (CAUSAL) top = min(top, qrow - k0);
            int lo = 0;
            if constexpr (WIN) {
                if (p.wr >= 0) top = min(top, qrow + p.wr - k0);
                if (p.wl >= 0) lo = qrow - p.wl - k0 - hi * 8;
            }
            top -= hi * 8;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = kb * 32 + (i >> 3) * 16 + (i & 7);
                    bool keep = c <= top;
                    if constexpr (WIN) keep = keep && c >= lo;
                    st[kb][i] = keep ? st[kb][i] : -INFINITY;
                }
        }
        // Stabiliser: the running max is moved to the true max only when it
        // has to be.  p = exp2(s*c - m*c) is first formed with the current
        // m; only if some lane's partial row sum exceeds kPpSumBound = 2^15
        // (so a single p might, and the fp16 range would be at risk) is m
        // raised to the row max, the accumulator rescaled and the tile's p
        // formed again (bf16: pp_headroom orders above the max).  In exact
        // arithmetic the softmax does not depend on the stabiliser (l and
        // the accumulator share it); in bf16 the largest p is then not a
        // power of two, so O is divided by the sum of the rounded p (see
        // Bf16Ops).  p stays at or below 2^15.  Until a row has seen a key
        // (m = -inf) its first pass overflows (kPpUnseen) and the max is
        // taken.
        auto to_max = [&]() {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) m4[i & 3] = fmaxf(m4[i & 3], st[kb][i]);
            const float mx = half_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
            const float m_new = fmaxf(m_run, mx + head);
            // m_run = -inf gives alpha = 0 (nothing accumulated yet)
            const float alpha =
                (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            l_part *= alpha;
            if constexpr (Ops::kRoundedNorm) l_rnd *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        };
        // p of the tile (rounded into pk) and this lane's partial row sums
        // (fp32 in the result, rounded p in rr); the slot's loads are spread
        // over the first pass
        float rr;
        auto probs = [&](bool loads) {
            const float mc = (m_run == -INFINITY) ? -kPpUnseen : m_run * c;
            float r4[4], r2[2];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if (loads) {
#pragma unroll
                    for (int r = 0; r < LOADS; ++r)
                        if (kc == r * KC / LOADS) issue(pl, r);
                }
                const int kb = kc >> 1, h = kc & 1;
                float e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    e[i] = __builtin_amdgcn_exp2f(fmaf(st[kb][h * 8 + i], c, -mc));
                    if constexpr (!Ops::kSumRounded)
                        r4[i & 3] = kc == 0 && i < 4 ? e[i] : r4[i & 3] + e[i];
                }
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pk[kc][w] = Ops::pack2(e[2 * w], e[2 * w + 1]);
                    if constexpr (Ops::kRoundedNorm || Ops::kSumRounded)
                        r2[w & 1] = Ops::add2(pk[kc][w], kc == 0 && w < 2 ? 0.f : r2[w & 1]);
                }
            }
            if constexpr (Ops::kRoundedNorm) rr = r2[0] + r2[1];
            if constexpr (Ops::kSumRounded) return r2[0] + r2[1];
            return (r4[0] + r4[1]) + (r4[2] + r4[3]);
        };
        // (one rescale site: a second branch around the accumulator made the
        // register allocator copy it on the common path)
        float r = probs(true);
        if (__any(r > kPpSumBound)) {   // rare (and a row's first visible tile)
            to_max();
            r = probs(false);
        }
        l_part += r;
        if constexpr (Ops::kRoundedNorm) l_rnd += rr;
        // P must exist before the barrier
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) __asm__ volatile("" : "+v"(pk[kc]));
    };
    // End of slot t: wait for all loads but this slot's, then a barrier.
    // Group 1 ends on an MFMA phase in slot 2*ntiles + 1, after which no
    // barrier is needed.
    const int last_slot = 2 * ntiles + 1;
    auto slot_end = [&](int t) {
        wait_vmcnt<LOADS>();
        if (t != last_slot) __syncthreads();
    };

    // A block whose rows see no key (possible only with a window) skips the
    // whole slot sequence, barriers included (the test is the same for every
    // wave), and stores O = 0, LSE = -inf.
    if (!WIN || ntiles > 0) {
        // Loads per slot: group 0 runs SM_j in slot 2j+1 (loads K_{j+2}) and
        // PV_j+QK_{j+1} in slot 2j+2 (loads V_{j+2}); group 1 runs SM_j in slot
        // 2j+2 (V_{j+2}) and PV_j+QK_{j+1} in slot 2j+3 (K_{j+3}).
        {
            const LoadPlan k0p = plan_kv(true, 0), v0p = plan_kv(false, 0), k1p = plan_kv(true, 1);
#pragma unroll
            for (int r = 0; r < LOADS; ++r) {
                issue(k0p, r);
                issue(v0p, r);
                issue(k1p, r);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
        int t = 0;
        if (grp == 1) {   // group 1 starts one slot late, loading its share of V_1
            const LoadPlan pl = plan(false, 1, ld_sm);
#pragma unroll
            for (int r = 0; r < LOADS; ++r) issue(pl, r);
            slot_end(t);
            ++t;
        }
        {   // S^T of tile 0 (loads V_1 in group 0's slot 0, K_2 in group 1's slot 1)
            const LoadPlan pl = plan(grp == 1, 1 + grp, ld_mf);
#pragma unroll
            for (int dc = 0; dc < DC; ++dc)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) qk_mma(k_lds[0], dc, kb);
#pragma unroll
            for (int r = 0; r < LOADS; ++r) issue(pl, r);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" : "+v"(st[kb]));
            slot_end(t);
            ++t;
        }
        // unrolled by three so that every LDS read address is a constant offset
        auto tile = [&](int j, const uint8_t *vbuf, const uint8_t *kbuf) {
            {
                const LoadPlan pl = plan(grp == 0, j + 2, ld_sm);
                softmax(pl, j);
                slot_end(t);
                ++t;
            }
            {
                const LoadPlan pl = plan(grp == 1, j + 2 + grp, ld_mf);
                mfma_phase(pl, vbuf, kbuf);
                slot_end(t);
                ++t;
            }
        };
        for (int j = 0; j < ntiles; j += 3) {
            tile(j, v_lds[0], k_lds[1]);
            if (j + 1 >= ntiles) break;
            tile(j + 1, v_lds[1], k_lds[2]);
            if (j + 2 >= ntiles) break;
            tile(j + 2, v_lds[2], k_lds[0]);
        }
        // no load may still be writing LDS when the workgroup ends
        wait_vmcnt<0>();
    }

    // ---- epilogue: O = acc / l, rounded to nearest even; LSE = m*scale + ln l.
    // Every wave past its last LDS read and load (the barrier), each wave's
    // 32 rows of O pass through its own 32 rows' worth of the K/V buffers
    // (waves 0-3 in the K buffers, 4-7 in the V buffers), so that the stores
    // to HBM are whole rows: 16 bytes per lane and four rows of O per
    // instruction, instead of 8-byte pieces scattered over 32 rows.  (The
    // next workgroup on this CU needs the whole LDS allocation, so waiting
    // here for the later wave group delays nothing.)
    const float l = half_sum(l_part);
    const float ln = Ops::kRoundedNorm ? half_sum(l_rnd) : l;
    const float inv = ln > 0.f ? 1.f / ln : 0.f;
    __syncthreads();
    uint32_t ob = (wave < 4 ? k_base : v_base) + (uint32_t)((wave & 3) * 32 * ROWB);
    {
        const uint32_t orow = (uint32_t)(l32 * ROWB);
        const int sw = swz_k<D>(l32);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // elements db*32 + g*8 + hi*4 .. +3: 16-byte chunk db*4 + g
                u32x2 x = {Ops::pack2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                           Ops::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                ds_store_b64_opaque(ob, orow + (uint32_t)(((db * 4 + g) ^ sw) * 16 + hi * 8), x);
            }
    }
    constexpr int OPIECES = 32 * KCH / 64;   // 16-byte pieces per lane
#pragma unroll
    for (int i = 0; i < OPIECES; ++i) {
        const int idx = i * 64 + lane, rr = idx / KCH, cc = idx % KCH;
        const u32x4 val = lds_load_b128(ob + (uint32_t)(rr * ROWB + ((cc ^ swz_k<D>(rr)) * 16)));
        if (qw + rr < p.Lq)
            *reinterpret_cast<u32x4 *>(p.o + og_base + (int64_t)(qw + rr) * o_sl + cc * 8) = val;
    }
    if (p.lse != nullptr && hi == 0 && qrow < p.Lq)
        p.lse[(int64_t)bh * p.Lq + qrow] = l > 0.f ? m_run * p.scale + __logf(l) : -INFINITY;
}

template <typename Ops, int D, bool CAUSAL, int BN, bool GEN = false, bool WIN = false>
hipError_t launch_pp(const FwdArgs &a)
{
    constexpr int BM = 256;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + BM - 1) / BM);
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    p.H = (int)a.H;
    p.wl = a.wl;
    p.wr = a.wr;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = a.qs[i];
        p.ks[i] = a.ks[i];
        p.vs[i] = a.vs[i];
        p.os[i] = a.os[i];
    }
    const int64_t nwg = (int64_t)p.BH * p.ntq;
    hipLaunchKernelGGL((fa_fwd_mfma_pp_kernel<Ops, D, CAUSAL, BN, GEN, WIN>), dim3((unsigned)nwg),
                       dim3(512), 0, a.stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Persistent ping-pong kernel (pipe 5; contiguous, non-causal, 64-key tiles).
//
// The ping-pong kernel (below, pipe 3) pays a fixed cost per workgroup: the
// first loads and their wait, one idle slot of the second wave group, the
// discarded first softmax pass and the epilogue, about 15,000 shader cycles
// in all, or 7% of a workgroup at the mid shape (cycle stamps of every phase
// of every wave on the part).  Here one workgroup per CU runs the query
// blocks g, g + G, g + 2G, ... (G = grid size, a multiple of 8, so that every
// block runs on the XCD that decompose() gives it) as one stream of key
// tiles: the slots of the ping-pong schedule run on from the last tile of one
// block into the first tile of the next, so loads, QK^T and softmax of the
// next block overlap the end of the previous one.  Per block boundary:
//   * the next block's Q rows are loaded into an LDS stage (64 KB) while the
//     block's second tile is processed, and copied into the Q^T registers in
//     the softmax slot of its last tile, right before the MFMA phase that
//     computes S of the next block's first tile;
//   * the softmax slot of a block's first tile first stores the previous
//     block's O and LSE and resets the row state (the accumulator holds the
//     previous block's last P.V, issued in the slot before).
// Every tile, block and slot otherwise follows the ping-pong kernel.
// ---------------------------------------------------------------------------
template <typename Ops, int D, int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_mfma_pers_kernel(Params p)
{
    constexpr int NW = 8;
    constexpr int BM = NW * 32;          // query rows per block
    constexpr int DC = D / 16;           // 16-dim chunks (k of the QK^T MFMA)
    constexpr int DB = D / 32;           // 32-dim blocks (rows of O^T)
    constexpr int KB = BN / 32;          // 32-key blocks (rows of S^T)
    constexpr int KC = BN / 16;          // 16-key chunks (k of the PV MFMA)
    constexpr int ROWB = D * 2;          // bytes per K, V or Q row in LDS
    constexpr int KCH = D / 8;           // 16-byte chunks per row
    constexpr int TILEB = BN * ROWB;     // bytes of one K (or V) tile
    constexpr int QB_BYTES = BM * ROWB;  // bytes of the Q stage
    constexpr int LOADS = TILEB / (NW * 64 * 16);      // loads per wave per tile
    constexpr int QL = QB_BYTES / (NW * 64 * 16);      // loads per wave per Q stage
    static_assert(LOADS >= 1 && TILEB % (NW * 64 * 16) == 0, "tile split");
    static_assert(6 * TILEB + QB_BYTES <= 160 * 1024, "K, V buffers and the Q stage fit the LDS");

    // one LDS array carved by hand: K and V buffers at the bottom, as in the
    // ping-pong kernel, so their reads keep constant offsets that fit the
    // 16-bit offset field; the Q stage on top
    __shared__ __attribute__((aligned(1024))) uint8_t lds[6 * TILEB + QB_BYTES];
    uint8_t(*k_lds)[TILEB] = reinterpret_cast<uint8_t(*)[TILEB]>(lds);
    uint8_t(*v_lds)[TILEB] = reinterpret_cast<uint8_t(*)[TILEB]>(lds + 3 * TILEB);
    uint8_t *q_lds = lds + 6 * TILEB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;           // waves w and w+4 share a SIMD
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // ---- the blocks of this workgroup and the tile stream
    const int nwg = p.BH * p.ntq;
    const int G = gridDim.x, g = blockIdx.x;
    const int nitems = (nwg - g + G - 1) / G;    // >= 1: G <= nwg
    const int n = (p.Lk + BN - 1) / BN;          // tiles per block (>= 4, host-checked)
    const int T = nitems * n;                    // tiles in the stream
    auto item = [&](int r, int &bh, int &q_first) {
        int qt;
        decompose(g + r * G, nwg, p.BH, p.ntq, false, bh, qt);
        q_first = qt * BM;
    };
    // current block r (of the tile being processed), the next one, and the
    // one whose output is still to be stored
    int bh_cur, qf_cur, bh_nxt = 0, qf_nxt = 0, bh_prev = 0, qf_prev = 0;
    item(0, bh_cur, qf_cur);
    if (nitems > 1) item(1, bh_nxt, qf_nxt);

    const int64_t seqk = (int64_t)p.Lk * D;      // elements per (b, h) of K and V
    const int64_t seqq = (int64_t)p.Lq * D;      // elements per (b, h) of Q and O

    // ---- Q^T operand of the first block in VGPRs (rows past Lq read the
    // last row and are never stored)
    u32x4 qreg[DC];
    {
        const int row = min(qf_cur + wave * 32 + l32, p.Lq - 1);
        const uint16_t *qh = p.q + (int64_t)bh_cur * seqq;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            qreg[dc] = *reinterpret_cast<const u32x4 *>(qh + (int64_t)((uint32_t)row * D) +
                                                        dc * 16 + hi * 8);
    }

    // ---- loads (as the ping-pong kernel): per-lane source offsets of this
    // wave's pieces; softmax phases load one tensor, MFMA phases the other
    int ld_row[LOADS];
    uint32_t ld_sm[LOADS], ld_mf[LOADS];
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
        const int sl = (r * NW + wave) * 64 + lane;
        const int row = sl / KCH, pc = sl % KCH;
        ld_row[r] = row;
        const uint32_t ov = (uint32_t)(row * D + (pc ^ swz_v<D>(row)) * 8) * 2;
        const uint32_t ok = (uint32_t)(row * D + (pc ^ swz_k<D>(row)) * 8) * 2;
        ld_sm[r] = grp == 0 ? ok : ov;
        ld_mf[r] = grp == 0 ? ov : ok;
    }
    const uint32_t k_base = lds_addr(k_lds[0]), v_base = lds_addr(v_lds[0]);
    struct LoadPlan {
        const uint16_t *src;
        uint32_t dst;
        uint32_t off[LOADS];
    };
    // the block of the tile being processed (r, local tile lt) and the
    // element offsets of the current and the next block within K and V
    int r = 0, lt = 0;
    int64_t base_cur = (int64_t)bh_cur * seqk, base_nxt = (int64_t)bh_nxt * seqk;
    // Element offset of the tile at local index la of the current block's
    // stream (la >= n: tile la - n of the next block; past the end of the
    // stream the last tile is fetched again, into a buffer no wave reads any
    // more) and the last valid key row in it (BN - 1 or more: a whole tile).
    auto locate = [&](int la, int64_t &off, int &last) {
        int64_t base = base_cur;
        int lk = la;
        if (la >= n) {
            if (r + 1 < nitems) {
                base = base_nxt;
                lk = la - n;
            } else {
                lk = n - 1;
            }
        }
        off = base + (int64_t)(lk * BN) * D;
        last = p.Lk - 1 - lk * BN;
    };
    // the loads of one phase into the buffer at byte offset buf_off (rows
    // past the last valid key fetch that row, as in the ping-pong kernel)
    auto make_plan = [&](bool is_k, int64_t off, int last, uint32_t buf_off,
                         const uint32_t (&whole)[LOADS]) {
        LoadPlan pl;
        pl.src = (is_k ? p.k : p.v) + off;
        pl.dst = (is_k ? k_base : v_base) + buf_off + (uint32_t)(wave * 1024);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) pl.off[q] = whole[q];
        if (last < BN - 1) {
#pragma unroll
            for (int q = 0; q < LOADS; ++q)
                pl.off[q] -= (uint32_t)max(ld_row[q] - last, 0) * (uint32_t)(D * 2);
        }
        return pl;
    };
    auto issue = [&](const LoadPlan &pl, int r) {
        dma_16B_sbase(pl.src, pl.off[r], pl.dst + (uint32_t)(r * NW * 1024));
    };
    // The next block's Q rows into the LDS stage: row i of the block at
    // byte i * ROWB, 16-byte chunks XOR-swizzled by row as in the K tiles.
    // (The rare paths below take the lane index through an opaque copy, so
    // that their addresses are formed when they run rather than hoisted out
    // of the tile loop into registers held across it.)
    auto opaque_lane = [&]() {
        int x = lane;
        __asm__ volatile("" : "+v"(x));
        return x;
    };
    auto stage_q = [&]() {
        const uint16_t *qh = p.q + (int64_t)bh_nxt * seqq;
        const uint32_t dst = lds_addr(q_lds) + (uint32_t)(wave * 1024);
        const int ln_ = opaque_lane();
#pragma unroll
        for (int r = 0; r < QL; ++r) {
            const int sl = (r * NW + wave) * 64 + ln_;
            const int row = sl / KCH, pc = sl % KCH;
            const int src_row = min(qf_nxt + row, p.Lq - 1);
            const uint32_t off = (uint32_t)(src_row * D + (pc ^ swz_k<D>(row)) * 8) * 2;
            dma_16B_sbase(qh, off, dst + (uint32_t)(r * NW * 1024));
        }
    };
    auto load_q_from_stage = [&]() {
        const int ln_ = opaque_lane();
        const int row = wave * 32 + (ln_ & 31);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            qreg[dc] = *reinterpret_cast<const u32x4 *>(
                q_lds + row * ROWB + (((dc * 2 + (ln_ >> 5)) ^ swz_k<D>(row)) * 16));
    };

    // ---- per-lane LDS read offsets (loop invariant)
    uint32_t k_rd[DC];
    {
        const int row = swap_bits23(l32);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            k_rd[dc] = (uint32_t)(row * ROWB + (((dc * 2 + hi) ^ swz_k<D>(row)) * 16));
    }
    // V read addresses in LDS, absolute (base of V buffer 0 included): the
    // V buffers end above 64 KB, and with the base folded into the register
    // every read of every buffer keeps an immediate offset below 64 KB
    // (buffer * TILEB + key chunk), where a buffer-relative register would
    // need an add before each read of buffers 1 and 2
    uint32_t v_rd[DB];
    {
        const int gq = lane >> 4, t = lane & 15;
        const int row = 8 * hi + (t >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (gq & 1) + 4 * (t & 3);
            const int cc = col >> 3, within = (col & 7) * 2;
            v_rd[db] = v_base + (uint32_t)(row * ROWB + ((cc ^ swz_v<D>(row)) * 16) + within);
            __asm__ volatile("" : "+v"(v_rd[db]));
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_part = 0.f, l_rnd = 0.f;
    const float c = p.c;
    const float head = pp_headroom<Ops>() / c;

    f32x16 st[KB];
    u32x4 pk[KC];

    auto qk_mma = [&](const uint8_t *kbuf, int dc, int kb) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(kbuf + k_rd[dc] + kb * 32 * ROWB);
        if (dc == 0) {
            f32x16 z;
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = 0.f;
            st[kb] = Ops::mma(a, qreg[0], z);
        } else {
            st[kb] = Ops::mma(a, qreg[dc], st[kb]);
        }
    };
    constexpr int NPV = KC * DB, NQK = DC * KB;
    auto read_v = [&](int vb, int kc, int db) {
        const uint32_t a = v_rd[db] + (uint32_t)(vb * TILEB + kc * 16 * ROWB);
        const uint2 lo = ds_read_tr_at(a);
        const uint2 hi4 = ds_read_tr_at(a + 4 * ROWB);
        return u32x4{lo.x, lo.y, hi4.x, hi4.y};
    };
    auto load_at = [](int r) { return 2 + r * ((NPV + NQK) / LOADS); };
    // the MFMA phase of the ping-pong kernel
    auto mfma_phase = [&](const LoadPlan &pl, int vb, const uint8_t *kbuf) {
        if (PP_PRIO) __builtin_amdgcn_s_setprio(PP_PRIO);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 a = read_v(vb, kc, db);
                oacc[db] = Ops::mma(a, pk[kc], oacc[db]);
#pragma unroll
                for (int r = 0; r < LOADS; ++r)
                    if (kc * DB + db == load_at(r)) issue(pl, r);
            }
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                qk_mma(kbuf, dc, kb);
#pragma unroll
                for (int r = 0; r < LOADS; ++r)
                    if (NPV + dc * KB + kb == load_at(r)) issue(pl, r);
            }
        constexpr int LEAD = PP_LEAD;
        constexpr int NM = NPV + NQK;
        static_assert(LEAD >= 1 && LEAD <= NPV, "read lead");
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
#pragma unroll
        for (int nn = 0; nn < NPV - LEAD; ++nn) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int nn = NPV - LEAD; nn < NM - LEAD; ++nn) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
        if (PP_PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" : "+v"(st[kb]));
    };
    // the softmax phase of the ping-pong kernel for local tile lt
    auto softmax = [&](const LoadPlan &pl, int lt) {
        const int k0 = lt * BN;
        if (k0 + BN > p.Lk) {
            int top = p.Lk - 1 - k0 - hi * 8;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int cc = kb * 32 + (i >> 3) * 16 + (i & 7);
                    st[kb][i] = cc <= top ? st[kb][i] : -INFINITY;
                }
        }
        auto to_max = [&]() {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) m4[i & 3] = fmaxf(m4[i & 3], st[kb][i]);
            const float mx = half_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
            const float m_new = fmaxf(m_run, mx + head);
            const float alpha =
                (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            l_part *= alpha;
            if constexpr (Ops::kRoundedNorm) l_rnd *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        };
        float rr;
        auto probs = [&](bool loads) {
            const float mc = (m_run == -INFINITY) ? -kPpUnseen : m_run * c;
            float r4[4], r2[2];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if (loads) {
#pragma unroll
                    for (int r = 0; r < LOADS; ++r)
                        if (kc == r * KC / LOADS) issue(pl, r);
                }
                const int kb = kc >> 1, h = kc & 1;
                float e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    e[i] = __builtin_amdgcn_exp2f(fmaf(st[kb][h * 8 + i], c, -mc));
                    if constexpr (!Ops::kSumRounded)
                        r4[i & 3] = kc == 0 && i < 4 ? e[i] : r4[i & 3] + e[i];
                }
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pk[kc][w] = Ops::pack2(e[2 * w], e[2 * w + 1]);
                    if constexpr (Ops::kRoundedNorm || Ops::kSumRounded)
                        r2[w & 1] = Ops::add2(pk[kc][w], kc == 0 && w < 2 ? 0.f : r2[w & 1]);
                }
            }
            if constexpr (Ops::kRoundedNorm) rr = r2[0] + r2[1];
            if constexpr (Ops::kSumRounded) return r2[0] + r2[1];
            return (r4[0] + r4[1]) + (r4[2] + r4[3]);
        };
        float r = probs(true);
        if (__any(r > kPpSumBound)) {   // rare (and a block's first tile)
            to_max();
            r = probs(false);
        }
        l_part += r;
        if constexpr (Ops::kRoundedNorm) l_rnd += rr;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) __asm__ volatile("" : "+v"(pk[kc]));
    };
    // O = acc / l rounded to nearest even and LSE of block (bh, q_first).
    // The wave's 32 rows pass through its own 8 KB of the Q stage (free at
    // a block's first tile: the block's Q is in registers, the next block's
    // is staged one tile later), so that the stores to HBM are whole rows,
    // 16 bytes per lane and four rows (1 KB of O) per instruction, instead
    // of 8-byte pieces scattered over 32 rows.
    auto epilogue = [&](int bh, int q_first) {
        const float l = half_sum(l_part);
        const float ln = Ops::kRoundedNorm ? half_sum(l_rnd) : l;
        const float inv = ln > 0.f ? 1.f / ln : 0.f;
        const int ln_ = opaque_lane();
        const int e32 = ln_ & 31, ehi = ln_ >> 5;
        uint32_t ow = lds_addr(q_lds) + (uint32_t)(wave * (32 * ROWB));
        {
            const uint32_t orow = (uint32_t)(e32 * ROWB);
            const int sw = swz_k<D>(e32);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    // elements db*32 + gg*8 + hi*4 .. +3: 16-byte chunk db*4 + gg
                    u32x2 x = {Ops::pack2(oacc[db][4 * gg] * inv, oacc[db][4 * gg + 1] * inv),
                               Ops::pack2(oacc[db][4 * gg + 2] * inv, oacc[db][4 * gg + 3] * inv)};
                    ds_store_b64_opaque(ow, orow + (uint32_t)(((db * 4 + gg) ^ sw) * 16 + ehi * 8), x);
                }
        }
        const int row0 = q_first + wave * 32;
        uint16_t *obase = p.o + (int64_t)bh * seqq;
        constexpr int OPIECES = 32 * KCH / 64;   // 16-byte pieces per lane
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < OPIECES; ++i) {
            const int idx = i * 64 + ln_, rr = idx / KCH, cc = idx % KCH;
            const u32x4 val =
                lds_load_b128(ow + (uint32_t)(rr * ROWB + ((cc ^ swz_k<D>(rr)) * 16)));
            if (row0 + rr < p.Lq)
                *reinterpret_cast<u32x4 *>(obase + (int64_t)(row0 + rr) * D + cc * 8) = val;
            if (i % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
        if (p.lse != nullptr && ehi == 0 && row0 + e32 < p.Lq)
            p.lse[(int64_t)bh * p.Lq + row0 + e32] =
                l > 0.f ? m_run * p.scale + __logf(l) : -INFINITY;
    };
    const int last_slot = 2 * T + 1;
    // End of slot t: every load but this slot's has landed (the Q stage and
    // the stores of an epilogue are issued before the slot's tile loads),
    // then a barrier; none after group 1's final MFMA phase.
    auto slot_end = [&](int t) {
        wait_vmcnt<LOADS>();
        if (t != last_slot) __syncthreads();
    };

    // ---- prologue: K_0, V_0, K_1 of the first block
    {
        int64_t o0, o1;
        int l0, l1;
        locate(0, o0, l0);
        locate(1, o1, l1);
        const LoadPlan k0p = make_plan(true, o0, l0, 0, (grp == 0) ? ld_sm : ld_mf);
        const LoadPlan v0p = make_plan(false, o0, l0, 0, (grp == 0) ? ld_mf : ld_sm);
        const LoadPlan k1p = make_plan(true, o1, l1, TILEB, (grp == 0) ? ld_sm : ld_mf);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            issue(k0p, q);
            issue(v0p, q);
            issue(k1p, q);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    int t = 0;
    if (grp == 1) {   // group 1 starts one slot late, loading its share of V_1
        int64_t o1;
        int l1;
        locate(1, o1, l1);
        const LoadPlan pl = make_plan(false, o1, l1, TILEB, ld_sm);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) issue(pl, q);
        slot_end(t);
        ++t;
    }
    {   // S^T of tile 0 (loads V_1 in group 0's slot 0, K_2 in group 1's slot 1)
        int64_t o;
        int l;
        locate(1 + grp, o, l);
        const LoadPlan pl = make_plan(grp == 1, o, l, (uint32_t)((1 + grp) * TILEB), ld_mf);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qk_mma(k_lds[0], dc, kb);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) issue(pl, q);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" : "+v"(st[kb]));
        slot_end(t);
        ++t;
    }

    // Stream tile j (j % 3 == B) of block r at local tile lt.  The loads of
    // a slot are for stream tiles j + 2 (softmax phase) and j + 2 + grp
    // (MFMA phase).  Within a block they advance by one tile per tile; the
    // first two and the last three tiles of a block (where a load or the
    // rows change block) take one branch that does the block's boundary
    // work and places the loads afresh.
    int64_t off_sm = 0, off_mf = 0;   // tiles loaded in the softmax and MFMA phases
    int last_sm = BN, last_mf = BN;
    auto tile = [&](auto bc, const uint8_t *kbuf) {
        constexpr int B = decltype(bc)::value;
        // softmax phase
        {
            if (lt < 2 || lt + 3 >= n) {
                if (lt == n) {   // the next block
                    lt = 0;
                    ++r;
                    bh_prev = bh_cur;
                    qf_prev = qf_cur;
                    bh_cur = bh_nxt;
                    qf_cur = qf_nxt;
                    base_cur = base_nxt;
                    if (r + 1 < nitems) {
                        item(r + 1, bh_nxt, qf_nxt);
                        base_nxt = (int64_t)bh_nxt * seqk;
                    }
                }
                if (lt == 1 && r + 1 < nitems) stage_q();
                locate(lt + 2, off_sm, last_sm);
                locate(lt + 2 + grp, off_mf, last_mf);
            } else {
                off_sm += BN * D;
                off_mf += BN * D;
            }
            // (the two rare steps below sit outside the branch above: inside
            // it they raise the register count of the whole loop)
            if (lt == 0 && r > 0) {   // store the previous block, reset the rows
                epilogue(bh_prev, qf_prev);
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
                m_run = -INFINITY;
                l_part = 0.f;
                l_rnd = 0.f;
            }
            const LoadPlan pl =
                make_plan(grp == 0, off_sm, last_sm, (uint32_t)(((B + 2) % 3) * TILEB), ld_sm);
            softmax(pl, lt);
            // Q of the next block: its first S^T is formed in this tile's
            // MFMA phase
            if (lt == n - 1 && r + 1 < nitems) load_q_from_stage();
            slot_end(t);
            ++t;
        }
        // MFMA phase: P V of this tile, S of the next (of the next block at
        // the block's last tile)
        {
            const uint32_t bo = grp ? (uint32_t)(B * TILEB) : (uint32_t)(((B + 2) % 3) * TILEB);
            const LoadPlan pl = make_plan(grp == 1, off_mf, last_mf, bo, ld_mf);
            mfma_phase(pl, B, kbuf);
            slot_end(t);
            ++t;
        }
        ++lt;
    };
    for (int j = 0; j < T; j += 3) {
        tile(std::integral_constant<int, 0>{}, k_lds[1]);
        if (j + 1 >= T) break;
        tile(std::integral_constant<int, 1>{}, k_lds[2]);
        if (j + 2 >= T) break;
        tile(std::integral_constant<int, 2>{}, k_lds[0]);
    }
    // no load may still be writing LDS when the workgroup ends
    wait_vmcnt<0>();
    epilogue(bh_cur, qf_cur);
}

template <typename Ops, int D, int BN>
hipError_t launch_pers(const FwdArgs &a, int grid)
{
    constexpr int BM = 256;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + BM - 1) / BM);
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    hipLaunchKernelGGL((fa_fwd_mfma_pers_kernel<Ops, D, BN>), dim3((unsigned)grid), dim3(512), 0,
                       a.stream, p);
    return hipGetLastError();
}

template <typename Ops, int D, bool CAUSAL, int NW, int QB, int BN, int OCC>
hipError_t launch_dma(const FwdArgs &a)
{
    constexpr int BM = NW * QB * 32;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + BM - 1) / BM);
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    const int64_t nwg = (int64_t)p.BH * p.ntq;
    hipLaunchKernelGGL((fa_fwd_mfma_dma_kernel<Ops, D, CAUSAL, NW, QB, BN, OCC>),
                       dim3((unsigned)nwg), dim3(NW * 64), 0, a.stream, p);
    return hipGetLastError();
}

template <typename Ops, int D, bool CAUSAL, int NW>
hipError_t launch_general_t(const FwdArgs &a)
{
    constexpr int BM = NW * 32;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + BM - 1) / BM);
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    p.H = (int)a.H;
    p.wl = a.wl;
    p.wr = a.wr;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = a.qs[i];
        p.ks[i] = a.ks[i];
        p.vs[i] = a.vs[i];
        p.os[i] = a.os[i];
    }
    const int64_t nwg = (int64_t)p.BH * p.ntq;
    hipLaunchKernelGGL((fa_fwd_mfma_dma_kernel<Ops, D, CAUSAL, NW, 1, 64, 2, true>),
                       dim3((unsigned)nwg), dim3(NW * 64), 0, a.stream, p);
    return hipGetLastError();
}

// The ping-pong kernel (96-key tiles at D = 128, 128-key tiles at D = 64)
// once there are 512 workgroups of 256 rows, as for contiguous calls.
template <typename Ops, bool WIN>
hipError_t launch_general_pp(const FwdArgs &a)
{
    if (a.D == 64)
        return a.causal ? launch_pp<Ops, 64, true, 128, true, WIN>(a)
                        : launch_pp<Ops, 64, false, 128, true, WIN>(a);
    constexpr int BN = WIN ? PP_WIN_BN : 96;
    return a.causal ? launch_pp<Ops, 128, true, BN, true, WIN>(a)
                    : launch_pp<Ops, 128, false, BN, true, WIN>(a);
}

// Smaller grids: 4 waves of the software-pipelined kernel (128 rows per
// workgroup, twice as many workgroups).
template <typename Ops>
hipError_t launch_general_ops(const FwdArgs &a)
{
    const bool big = a.B * a.H * ((a.Lq + 255) / 256) >= 512;
    if (big && GENERAL_PP)
        return (a.wl >= 0 || a.wr >= 0) ? launch_general_pp<Ops, true>(a)
                                        : launch_general_pp<Ops, false>(a);
    if (a.D == 64) {
        if (a.causal) return big ? launch_general_t<Ops, 64, true, 8>(a) : launch_general_t<Ops, 64, true, 4>(a);
        return big ? launch_general_t<Ops, 64, false, 8>(a) : launch_general_t<Ops, 64, false, 4>(a);
    }
    if (a.causal) return big ? launch_general_t<Ops, 128, true, 8>(a) : launch_general_t<Ops, 128, true, 4>(a);
    return big ? launch_general_t<Ops, 128, false, 8>(a) : launch_general_t<Ops, 128, false, 4>(a);
}

template <typename Ops, int D, bool CAUSAL, int NW, int QB, int BN, int OCC>
hipError_t launch_cfg(const FwdArgs &a)
{
    constexpr int BM = NW * QB * 32;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.ntq = (int)((a.Lq + BM - 1) / BM);
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    const int64_t nwg = (int64_t)p.BH * p.ntq;
    hipLaunchKernelGGL((fa_fwd_mfma_kernel<Ops, D, CAUSAL, NW, QB, BN, OCC>),
                       dim3((unsigned)nwg), dim3(NW * 64), 0, a.stream, p);
    return hipGetLastError();
}

template <typename Ops, int D, bool CAUSAL>
hipError_t launch_tile(const FwdArgs &a, const MfmaTile &t)
{
    if (t.nw == 4 && t.qb == 1 && t.bn == 64 && t.occ == 1)
        return launch_cfg<Ops, D, CAUSAL, 4, 1, 64, 1>(a);
    if (t.nw == 4 && t.qb == 1 && t.bn == 64 && t.occ == 2)
        return launch_cfg<Ops, D, CAUSAL, 4, 1, 64, 2>(a);
    if (t.nw == 8 && t.qb == 1 && t.bn == 64 && t.occ == 2)
        return launch_cfg<Ops, D, CAUSAL, 8, 1, 64, 2>(a);
    if (t.nw == 4 && t.qb == 2 && t.bn == 64 && t.occ == 1)
        return launch_cfg<Ops, D, CAUSAL, 4, 2, 64, 1>(a);
    return hipErrorInvalidConfiguration;
}

template <typename Ops, int D, bool CAUSAL>
hipError_t launch_tile_dma(const FwdArgs &a, const MfmaTile &t)
{
    if (t.nw == 8 && t.qb == 1 && t.bn == 64 && t.occ == 2)
        return launch_dma<Ops, D, CAUSAL, 8, 1, 64, 2>(a);
    if (t.nw == 4 && t.qb == 1 && t.bn == 64 && t.occ == 2)
        return launch_dma<Ops, D, CAUSAL, 4, 1, 64, 2>(a);
    if (t.nw == 4 && t.qb == 2 && t.bn == 64 && t.occ == 1)
        return launch_dma<Ops, D, CAUSAL, 4, 2, 64, 1>(a);
    // narrow workgroups (64 and 32 query rows): more workgroups on small
    // grids; in the tile sweep they lose to the 4-wave tile (latency bound)
    if (t.nw == 2 && t.qb == 1 && t.bn == 64 && t.occ == 1)
        return launch_dma<Ops, D, CAUSAL, 2, 1, 64, 1>(a);
    if (t.nw == 1 && t.qb == 1 && t.bn == 64 && t.occ == 1)
        return launch_dma<Ops, D, CAUSAL, 1, 1, 64, 1>(a);
    return hipErrorInvalidConfiguration;
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0 &&
        hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = 0;
    return cus[dev];
}

template <typename Ops>
hipError_t launch_ops(const FwdArgs &a, const MfmaTile &t)
{
    if (t.pipe == 5) {
        // persistent ping-pong kernel: D = 128, 64-key tiles, non-causal,
        // at least 4 tiles per block and one block per CU; grid = the CUs
        // (a multiple of 8), capped at the number of blocks
        const int64_t nwg = a.B * a.H * ((a.Lq + 255) / 256);
        const int64_t cus = device_cus();
        if (!(t.nw == 8 && t.qb == 1 && t.bn == 64 && t.occ == 2) || a.D != 128 || a.causal ||
            (a.Lk + 63) / 64 < 4 || cus < 8 || nwg < cus)
            return hipErrorInvalidConfiguration;
        return launch_pers<Ops, 128, 64>(a, (int)(cus / 8 * 8));
    }
    if (t.pipe == 3) {
        // 8 waves; 64-key tiles, 96-key tiles at D = 128 (six buffers of 24
        // KB), or 128-key tiles at D = 64 (six buffers of 32 KB would not
        // fit the LDS at D = 128)
        if (!(t.nw == 8 && t.qb == 1 && t.occ == 2)) return hipErrorInvalidConfiguration;
        if (a.D == 64) {
            if (t.bn == 128)
                return a.causal ? launch_pp<Ops, 64, true, 128>(a) : launch_pp<Ops, 64, false, 128>(a);
            if (t.bn == 64)
                return a.causal ? launch_pp<Ops, 64, true, 64>(a) : launch_pp<Ops, 64, false, 64>(a);
            return hipErrorInvalidConfiguration;
        }
        if (t.bn == 96)
            return a.causal ? launch_pp<Ops, 128, true, 96>(a) : launch_pp<Ops, 128, false, 96>(a);
        if (t.bn != 64) return hipErrorInvalidConfiguration;
        return a.causal ? launch_pp<Ops, 128, true, 64>(a) : launch_pp<Ops, 128, false, 64>(a);
    }
    if (t.pipe == 2) {
        if (a.D == 64)
            return a.causal ? launch_tile_dma<Ops, 64, true>(a, t)
                            : launch_tile_dma<Ops, 64, false>(a, t);
        return a.causal ? launch_tile_dma<Ops, 128, true>(a, t)
                        : launch_tile_dma<Ops, 128, false>(a, t);
    }
    if (a.D == 64)
        return a.causal ? launch_tile<Ops, 64, true>(a, t) : launch_tile<Ops, 64, false>(a, t);
    return a.causal ? launch_tile<Ops, 128, true>(a, t) : launch_tile<Ops, 128, false>(a, t);
}

}  // namespace

bool mfma_supported(const FwdArgs &a)
{
    return (a.dtype == 1 || a.dtype == 2) && (a.D == 64 || a.D == 128) && a.scale > 0.f;
}

MfmaTile mfma_choose_tile(const FwdArgs &a)
{
    // Static table from an offline sweep of every tile over shape classes
    // (scaled_dot_product_fa_amd/tune.py, timings in tiles.json), after one
    // rule for the persistent kernel (below).  Rules are per I/O type; the
    // bf16 and fp16 sweeps pick the same tiles.  In short: the ping-pong
    // kernel (8 waves, 256 query rows) once there are 512+ blocks of 256
    // rows and 2048+ visible keys per row (64-key tiles at D = 128
    // non-causal, 96-key causal, 128-key at D = 64); non-causal also from
    // 128 blocks (64-key tiles); otherwise 4 waves of the software-pipelined
    // kernel (128 rows per workgroup, twice as many workgroups).
    struct TileRule {
        int dtype, d, causal;
        int64_t min_blocks, min_kv;
        MfmaTile tile;
    };
    static const TileRule kRules[] = {
#include "fa_tiles.inc"
    };
    const int64_t blocks = a.B * a.H * ((a.Lq + 255) / 256);
    const int64_t kv = a.causal ? (a.Lk < a.Lq ? a.Lk : a.Lq) : a.Lk;
    // Ahead of the table: the persistent ping-pong kernel for short key
    // sequences (D = 128, non-causal, 4 to 32 key tiles) when every
    // workgroup gets at least two query blocks.  It saves most of the fixed
    // cost per query block, which is the larger share the shorter the row:
    // measured against the 64-key ping-pong kernel at 512 and 1024 blocks,
    // +7% to +9% at 256 keys, +4% at 512, +2% to +3% at 1024, +1% at 2048,
    // even at 3072 (its tiles cost about 0.8% more).
    if (a.D == 128 && !a.causal && a.Lk >= 4 * 64 - 63 && a.Lk <= 32 * 64) {
        const int64_t g = device_cus() / 8 * 8;
        if (g >= 8 && blocks >= 2 * g) return MfmaTile{8, 1, 64, 2, 5};
    }
    for (const TileRule &r : kRules)
        if (r.dtype == a.dtype && r.d == a.D && r.causal == (a.causal ? 1 : 0) &&
            blocks >= r.min_blocks && kv >= r.min_kv)
            return r.tile;
    return MfmaTile{4, 1, 64, 2, 2};
}

// Interned copy of a kernel label: the returned pointer stays valid for the
// life of the process and is the same for equal labels.
static const char *intern_name(const char *s)
{
    static std::mutex mu;
    static std::set<std::string> names;
    std::lock_guard<std::mutex> lock(mu);
    return names.insert(s).first->c_str();
}

// "fa_fwd_mfma_<dtype>_d<D>[_causal]_<family><waves>w[<QB>q]_bn<BN>", with
// family ppp (persistent ping-pong), pp (ping-pong), pipe (software-
// pipelined, LDS DMA) or reg (K/V staged through registers; "_occ<waves
// per SIMD>" appended).
const char *mfma_kernel_name(const FwdArgs &a, const MfmaTile &t)
{
    const char *fam = t.pipe == 5 ? "ppp" : t.pipe == 3 ? "pp" : t.pipe == 2 ? "pipe" : "reg";
    char buf[96];
    int n = snprintf(buf, sizeof buf, "fa_fwd_mfma_%s_d%d%s_%s%dw", a.dtype == 2 ? "bf16" : "f16",
                     (int)a.D, a.causal ? "_causal" : "", fam, t.nw);
    if (t.qb > 1) n += snprintf(buf + n, sizeof buf - n, "%dq", t.qb);
    n += snprintf(buf + n, sizeof buf - n, "_bn%d", t.bn);
    if (t.pipe == 0) snprintf(buf + n, sizeof buf - n, "_occ%d", t.occ);
    return intern_name(buf);
}

hipError_t mfma_launch(const FwdArgs &a, const MfmaTile &t)
{
    return a.dtype == 2 ? launch_ops<Bf16Ops>(a, t) : launch_ops<F16Ops>(a, t);
}

// As mfma_kernel_name, for the strided / windowed kernels that
// mfma_launch_general picks ("_strided", "_window" when a window is given).
const char *mfma_general_kernel_name(const FwdArgs &a)
{
    const bool big = a.B * a.H * ((a.Lq + 255) / 256) >= 512;
    const bool win = a.wl >= 0 || a.wr >= 0;
    MfmaTile t{big ? 8 : 4, 1, 64, 2, 2};
    if (big && GENERAL_PP) t = MfmaTile{8, 1, a.D == 64 ? 128 : (win ? PP_WIN_BN : 96), 2, 3};
    char buf[128];
    snprintf(buf, sizeof buf, "%s_strided%s", mfma_kernel_name(a, t), win ? "_window" : "");
    return intern_name(buf);
}

hipError_t mfma_launch_general(const FwdArgs &a)
{
    return a.dtype == 2 ? launch_general_ops<Bf16Ops>(a) : launch_general_ops<F16Ops>(a);
}

}  // namespace fa
