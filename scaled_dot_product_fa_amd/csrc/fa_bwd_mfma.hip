// fa_bwd_mfma.hip -- attention backward for gfx950 on bf16/fp16 MFMA.
//
// Gradients of O = softmax(scale Q K^T [+causal]) V for an incoming dO, by
// the chain rule through that definition, with the probabilities recomputed
// from the forward's row statistic lse rather than stored (the
// FlashAttention-2 forward article keeps Q, K, V, O and the statistic for the
// backward, and its account of the IO-aware idea notes that the backward may
// recompute instead of store):
//
//   p_ij = exp(scale q_i.k_j - lse_i),  ds_ij = p_ij (dO_i.v_j - delta_i),
//   dV_j = sum_i p_ij dO_i,  dK_j = scale sum_i ds_ij q_i,
//   dQ_i = scale sum_j ds_ij k_j,  delta_i = dO_i . O_i (computed beforehand).
//
// Two kernels, no atomics (so the result is deterministic):
//
//   * dK/dV kernel, one workgroup per block of keys.  Each wave owns 32 keys
//     and keeps their K and V rows in VGPRs as MFMA B operands.  Tiles of 32
//     query rows of Q and dO stream through LDS (direct global-to-LDS loads,
//     four buffers, software-pipelined).  Per tile: S = Q K^T and dP = dO V^T on
//     v_mfma_f32_32x32x16_{bf16,f16} with the Q/dO rows read in a permuted
//     order (bits 2 and 3 of the row swapped), so each lane's accumulator
//     holds one key column and two runs of 8 consecutive queries.  P and dS,
//     rounded to the I/O type, are then directly the B operands of
//     dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T come from the same LDS
//     tiles through ds_read_b64_tr_b16 (transposing reads).  At D = 128 (one
//     wave per SIMD, nothing else to fill the MFMA pipe's idle time) a step
//     forms S/dP of the next tile while the vector ALU turns the previous
//     step's S/dP into P and dS, then runs dV/dK; at D = 64 (two waves per
//     SIMD) the probabilities follow their own S/dP within a step.
//   * dQ kernel, one workgroup per block of query rows, the forward's layout:
//     each wave owns 32 queries with Q^T and dO^T in VGPRs; tiles of 64 keys
//     of K and V stream through LDS (direct loads, two buffers); S^T = K Q^T
//     and dP^T = V dO^T put one query column in each lane; dS^T is the B
//     operand of dQ^T += K^T dS^T, K^T read from the K tile with transposing
//     reads.
//
// The LDS tiles are row-major with 16-byte chunks XOR-swizzled by row with a
// pattern that keeps both the permuted row reads and the transposing reads
// free of bank conflicts.  exp uses exp2 with scale*log2(e) folded into one
// FMA.  Causal masking keeps key j for query i when j <= i: the dQ kernel
// skips key tiles a wave cannot see and masks only tiles that cross the
// diagonal; the dK/dV kernel starts at the first query tile that can see its
// keys and masks (rather than branches around) the few tiles a wave cannot
// see, so each pipeline step stays one straight-line block.
//
// Kernel variants: contiguous tensors (compile-time row strides), strided
// views (GEN: runtime strides), and strided views with the local window
// (GEN and WIN: query or key range clipped to the window, window edges
// masked).
//
// Compile-time knobs (defaults are the measured best): waves per SIMD each
// kernel is register-budgeted for, at D = 64 and D = 128 (BWD_*_OCC*), and
// whether the dK/dV step pins its MFMA / LDS-read / VALU interleave
// (BWD_KV_SCHED: sched_group_barrier with BWD_KV_VPER VALU ops per slot at
// two waves per SIMD, sched_barrier fences between the chunks at one).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

#ifndef BWD_KV_OCC64
#define BWD_KV_OCC64 2
#endif
#ifndef BWD_KV_OCC128
#define BWD_KV_OCC128 1
#endif
#ifndef BWD_KV_SCHED
#define BWD_KV_SCHED 1
#endif
#ifndef BWD_KV_VPER
#define BWD_KV_VPER 10
#endif
#ifndef BWD_Q_NW64
#define BWD_Q_NW64 4
#endif
#ifndef BWD_Q_NW128
#define BWD_Q_NW128 4
#endif
#ifndef BWD_Q_OCC64
#define BWD_Q_OCC64 2
#endif
#ifndef BWD_Q_OCC128
#define BWD_Q_OCC128 2
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;   // 4 waves per workgroup

struct Bf16Ops {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y)
    {
        bf16x2 r = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, r);
    }
};

struct F16Ops {
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
};

// Swap bits 2 and 3 of a row index within a 32-row block.  Reading A rows
// in this order makes accumulator element r of lane l belong to row
// 8*(l/32) + r (r < 8) or 16 + 8*(l/32) + (r - 8) (r >= 8).
__device__ __forceinline__ int swap_bits23(int r)
{
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Row index (0..31) of accumulator element r of a lane in half `hi`.
__device__ __forceinline__ int acc_row(int r, int hi)
{
    return r < 8 ? 8 * hi + r : 16 + 8 * hi + (r - 8);
}

// Chunk swizzle shared by every tile (64 LDS banks of 4 bytes).
//  * Permuted row reads (16 bytes per lane): a phase of 16 lanes reads rows
//    swap_bits23(0..15) at one logical chunk, so the swizzle must be a
//    bijection on rows mod 16 (D = 128, 256-byte rows) or, for D = 64
//    (128-byte rows, row parity picks the bank half), on the 8 rows of each
//    parity.
//  * Transposing reads (8 bytes per lane): a phase of 32 lanes reads 4
//    consecutive rows x 4 adjacent chunks; the 4 rows must land in distinct
//    4-chunk groups (D = 128), or rows r and r+2 must (D = 64).
// D = 128: f(r) = 4*(r%4) + (r/4)%4.  D = 64: x = (r/2)%8, f = 4*(x%2) + x/2.
template <int D>
__device__ __forceinline__ int swz(int row)
{
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
}

__device__ __forceinline__ uint2 ds_read_tr(const uint8_t *p)
{
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// global_load_lds_dwordx4 / _dword: every lane fetches 16 (4) bytes from its
// own global address and the hardware writes them to LDS at m0 + 16 (4) *
// lane.  Issued from inline assembly so that the compiler does not count
// them: it would otherwise wait for every outstanding LDS read before each
// use of any of them.  The kernels order them with explicit vmcnt waits and
// barriers, and drain them before exit.
__device__ __forceinline__ void dma_16B(const void *src, uint32_t lds_dst)
{
    __asm__ volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

__device__ __forceinline__ void dma_4B(const void *src, uint32_t lds_dst)
{
    __asm__ volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t uniform(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

struct BwdParams {
    const uint16_t *q, *k, *v, *dout;
    const float *lse, *delta;
    uint16_t *dq, *dk, *dv;
    int BH, Lq, Lk, nt;
    float scale, c;  // c = scale * log2(e)
    // strided / windowed calls only (GEN kernels): heads per batch, window
    // bounds (-1: none), element strides (batch, head, row) per tensor in
    // the order q, k, v, o, dout, dq, dk, dv
    int H, wl, wr;
    int64_t st[8][3];
};

// Per-(b, h) element base and row stride of tensor t: the contiguous
// [B, H, L, D] values unless GEN.
template <bool GEN, int D>
__device__ __forceinline__ void tensor_at(const BwdParams &p, int t, int bh, int L,
                                          int64_t &base, int &row_stride)
{
    if constexpr (GEN) {
        const int b = bh / p.H, h = bh % p.H;
        base = b * p.st[t][0] + h * p.st[t][1];
        row_stride = (int)p.st[t][2];
    } else {
        base = (int64_t)bh * L * D;
        row_stride = D;
    }
}

// Workgroup id -> (head bh, block t of nt per head).  Hardware places
// workgroup w on XCD w % 8; consecutive logical ids share an XCD, so one
// head's blocks (which stream the same tensors) share an L2.  Causal grids
// start with the longest blocks: low t when heavy_low, else high t.
__device__ __forceinline__ void decompose(int wg, int nwg, int BH, int nt, bool causal,
                                          bool heavy_low, int &bh, int &t)
{
    const int per = nwg >> 3, rem = nwg & 7;
    const int xcd = wg & 7, idx = wg >> 3;
    if (causal && (BH & 7) == 0) {
        const int hpx = BH >> 3;
        const int rank = idx / hpx;
        t = heavy_low ? rank : nt - 1 - rank;
        bh = xcd * hpx + idx % hpx;
        return;
    }
    const int logical = xcd < rem ? xcd * (per + 1) + idx
                                  : rem * (per + 1) + (xcd - rem) * per + idx;
    bh = logical / nt;
    t = logical % nt;
    if (causal && !heavy_low) t = nt - 1 - t;
}

// Per-lane LDS offsets of the transposing read: A operand [32 dims x 16
// rows] of block db, rows 8*hi..8*hi+3 (first read) and +4 (second read) of
// a 16-row chunk; add chunk * 16 * ROWB (the swizzle repeats every 16 rows).
template <int D, int DB>
__device__ __forceinline__ void tr_offsets(int lane, uint32_t (&off)[DB][2])
{
    constexpr int ROWB = D * 2;
    const int hi = lane >> 5, g = lane >> 4, t = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * hi + (t >> 2) + 4 * h;
            const int col = db * 32 + 16 * (g & 1) + 4 * (t & 3);
            const int c = col >> 3, within = (col & 7) * 2;
            off[db][h] = (uint32_t)(row * ROWB + ((c ^ swz<D>(row)) * 16) + within);
        }
}

template <int DB>
__device__ __forceinline__ u32x4 read_tr(const uint8_t *tile, const uint32_t (&off)[DB][2],
                                         int db, uint32_t chunk_off)
{
    const uint2 lo = ds_read_tr(tile + off[db][0] + chunk_off);
    const uint2 hi4 = ds_read_tr(tile + off[db][1] + chunk_off);
    return u32x4{lo.x, lo.y, hi4.x, hi4.y};
}

// An 8-byte LDS store the compiler does not see as one: an LDS store it
// knows of anywhere in a kernel makes it drop the read-ahead schedule of the
// MFMA steps.  `base` is an in-out operand, so every address formed from it
// afterwards follows the store (and a wave's LDS operations complete in
// issue order).
__device__ __forceinline__ void ds_store_b64_opaque(uint32_t &base, uint32_t off, uint2 v)
{
    __asm__ volatile("ds_write_b64 %1, %2" : "+v"(base) : "v"(base + off), "v"(v));
}

typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ u32x4 lds_load_b128(uint32_t a)
{
    return *(const lds_u32x4 *)(uintptr_t)a;
}

// A wave's 32 rows of gradient (the accumulator layout: lane l32 + 32*hi
// holds row l32, columns db*32 + 8g + 4hi .. +3 in acc[db][4g .. 4g+3]),
// times `mul`, rounded to the I/O type and stored as whole rows: through 32
// rows of this wave's own LDS at `stage` (16-byte chunk c of row r at
// position c ^ (r mod D/8)), then 16-byte pieces, four rows (D = 128) per
// store instruction instead of 8-byte pieces over 32 rows.  Rows >= nrows
// are not stored.
template <typename Ops, int D>
__device__ __forceinline__ void store_rows_staged(uint32_t stage, const f32x16 (&acc)[D / 32],
                                                  float mul, uint16_t *row0, int64_t row_stride,
                                                  int nrows, int lane)
{
    constexpr int ROWB = D * 2, CH = D / 8, DB = D / 32;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = Ops::pack2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul);
            w.y = Ops::pack2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
            ds_store_b64_opaque(
                stage, (uint32_t)(l32 * ROWB + (((db * 4 + g) ^ (l32 % CH)) * 16) + hi * 8), w);
        }
#pragma unroll
    for (int i = 0; i < 32 * CH / 64; ++i) {
        const int idx = i * 64 + lane, rr = idx / CH, cc = idx % CH;
        const u32x4 val = lds_load_b128(stage + (uint32_t)(rr * ROWB + ((cc ^ (rr % CH)) * 16)));
        if (rr < nrows) *(u32x4 *)(row0 + (int64_t)rr * row_stride + cc * 8) = val;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys, 32 per wave; query tiles of 32 rows,
// software-pipelined: in step t the S and dP products of tile t+1 and the
// dV, dK products of tile t are issued together, and the probabilities of
// tile t+1 are computed while the latter run.  Tiles reach LDS by direct
// loads (Q and dO rows, the 32 lse and 32 delta values) into four rotating
// buffers: tile t+3 is requested in step t and needed at the end of step
// t+1.  One barrier per step.  Causal tiles a wave cannot see are computed
// and masked to zero (no branch inside a step).
// ---------------------------------------------------------------------------
// GEN: runtime strides (strided views); WIN: the local window (with GEN).
template <typename Ops, int D, bool CAUSAL, int OCC, bool GEN = false, bool WIN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_bwd_dkdv_mfma_kernel(BwdParams p)
{
    constexpr int NW = kThreads / 64;
    constexpr int BK = NW * 32;
    constexpr int BQ = 32;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = BQ * ROWB;
    constexpr int NLD = BQ * CH / kThreads;     // 16-byte loads per lane per tensor
    constexpr int LPI = 2 * NLD + 1;            // loads per lane per tile
    constexpr int BUFB = 2 * TILEB + 2 * BQ * 4;
    constexpr int NBUF = 4;
    static_assert(NLD >= 1 && BQ * CH % kThreads == 0, "tile split");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * BUFB];
    static_assert(NW * 2 * 32 * ROWB <= NBUF * BUFB, "dK, dV staging fits the LDS");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    int bh, kt;
    decompose(blockIdx.x, gridDim.x, p.BH, p.nt, CAUSAL, true, bh, kt);
    const int Lq = p.Lq, Lk = p.Lk;
    const int k_first = kt * BK;
    const int kw = k_first + wave * 32;
    const int key = kw + l32;

    int64_t q_b, g_b, k_b, v_b, dk_b, dv_b;
    int q_sl, g_sl, k_sl, v_sl, dk_sl, dv_sl;
    tensor_at<GEN, D>(p, 0, bh, Lq, q_b, q_sl);
    tensor_at<GEN, D>(p, 4, bh, Lq, g_b, g_sl);
    tensor_at<GEN, D>(p, 1, bh, Lk, k_b, k_sl);
    tensor_at<GEN, D>(p, 2, bh, Lk, v_b, v_sl);
    tensor_at<GEN, D>(p, 6, bh, Lk, dk_b, dk_sl);
    tensor_at<GEN, D>(p, 7, bh, Lk, dv_b, dv_sl);
    const uint16_t *qh = p.q + q_b;
    const uint16_t *gh = p.dout + g_b;
    // lane l < 32 loads lse of row l of a tile, lane l >= 32 delta of row l-32
    const float *xh = (lane < 32 ? p.lse : p.delta) + (int64_t)bh * Lq;

    u32x4 kop[DC], vop[DC];
    {
        const uint16_t *kr = p.k + k_b + (int64_t)key * k_sl + 8 * hi;
        const uint16_t *vr = p.v + v_b + (int64_t)key * v_sl + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            kop[dc] = key < Lk ? *(const u32x4 *)(kr + dc * 16) : u32x4{0u, 0u, 0u, 0u};
            vop[dc] = key < Lk ? *(const u32x4 *)(vr + dc * 16) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dk[db][i] = 0.f;
            dv[db][i] = 0.f;
        }

    // Direct loads: load n of a wave fills the 1 KB at LDS chunk position
    // (n*NW + wave)*64 + lane of a tile; that position is row pos / CH,
    // physical chunk pos % CH, which holds logical chunk phys ^ swz(row).
    int dm_row[NLD];
    uint32_t dm_col[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int pos = (n * NW + wave) * 64 + lane;
        const int row = pos / CH, phys = pos % CH;
        dm_row[n] = row;
        dm_col[n] = (uint32_t)(((phys ^ swz<D>(row)) * 8));
    }
    const uint32_t smem_base = lds_addr(smem);
    // Rows past the end fetch the last row (valid memory); the probabilities
    // of those rows are masked to zero in the last step.
    auto issue = [&](int i0, uint32_t b) {
        const uint32_t wb = uniform(smem_base + b + (uint32_t)(wave * 1024));
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int64_t row = min(i0 + dm_row[n], Lq - 1);
            dma_16B(qh + row * q_sl + dm_col[n], wb + (uint32_t)(n * NW * 1024));
            dma_16B(gh + row * g_sl + dm_col[n], wb + TILEB + (uint32_t)(n * NW * 1024));
        }
        dma_4B(xh + min(i0 + l32, Lq - 1), uniform(smem_base + b + 2 * TILEB));
    };

    uint32_t rd_row[DC];
    {
        const int row = swap_bits23(l32);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            rd_row[dc] = (uint32_t)(row * ROWB + (((2 * dc + hi) ^ swz<D>(row)) * 16));
    }
    uint32_t rd_tr[DB][2];
    tr_offsets<D, DB>(lane, rd_tr);

    // query rows that see some key of the block: [i_begin, i_end)
    int i_begin = CAUSAL ? k_first : 0;
    int i_end = Lq;
    if constexpr (WIN) {
        if (p.wr >= 0) i_begin = max(i_begin, k_first - p.wr);
        if (p.wl >= 0) i_end = min(Lq, k_first + BK + p.wl);
        i_begin = max(i_begin, 0);
    }
    const int ntiles = i_begin < i_end ? (i_end - i_begin + BQ - 1) / BQ : 0;

    f32x16 s, dp;
    u32x4 pk[2], dsk[2];
    auto sdp = [&](uint32_t b) {
        u32x4 aq[DC], ag[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            aq[dc] = *(const u32x4 *)(smem + b + rd_row[dc]);
            ag[dc] = *(const u32x4 *)(smem + b + TILEB + rd_row[dc]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = 0.f;
            dp[i] = 0.f;
        }
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            s = Ops::mma(aq[dc], kop[dc], s);
            dp = Ops::mma(ag[dc], vop[dc], dp);
        }
    };
    // Probabilities and ds of the tile at rows i0.. (in LDS at b), in three
    // parts so that a step can spread them over its MFMAs: the row
    // statistics and mask bounds, one element, the packing.  TAIL: also
    // zero the rows past the end of the queries.
    struct PStat {
        float L[16], Dl[16];
        int lim, rows;
    };
    auto pstats = [&](uint32_t b, int i0) {
        PStat ps;
        // lse and delta of rows 8*hi + 0..7 and 16 + 8*hi + 0..7
        const float4 *lt4 = (const float4 *)(smem + b + 2 * TILEB) + 2 * hi;
        const float4 *dl4 = lt4 + BQ / 4;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int src = (q4 & 1) + 4 * (q4 >> 1);
            const float4 a = lt4[src], d = dl4[src];
            ps.L[4 * q4] = a.x; ps.L[4 * q4 + 1] = a.y; ps.L[4 * q4 + 2] = a.z; ps.L[4 * q4 + 3] = a.w;
            ps.Dl[4 * q4] = d.x; ps.Dl[4 * q4 + 1] = d.y; ps.Dl[4 * q4 + 2] = d.z; ps.Dl[4 * q4 + 3] = d.w;
        }
        // causal: keep key kw + l32 for row i0 + row when row >= lim
        int lim = (CAUSAL && i0 < kw + 31) ? kw + l32 - i0 : -1;
        int rows = Lq - i0;
        if constexpr (WIN) {
            // rows lim .. rows - 1 (relative to i0) keep this lane's key
            const int key_abs = kw + l32;
            if (p.wr >= 0) lim = max(lim, key_abs - p.wr - i0);
            if (p.wl >= 0) rows = min(rows, key_abs + p.wl + 1 - i0);
        }
        // element r is row 8*hi + c(r), c(r) = acc_row(r, 0) a constant
        ps.lim = lim - 8 * hi;
        ps.rows = rows - 8 * hi;
        return ps;
    };
    auto pelem = [&](const PStat &ps, int r, const f32x16 &s, const f32x16 &dp, float (&pv)[16],
                     float (&dsv)[16], auto tail) {
        float e = exp2_fast(fmaf(s[r], p.c, -ps.L[r] * kLog2e));
        if (CAUSAL || WIN) e = acc_row(r, 0) >= ps.lim ? e : 0.f;
        if (decltype(tail)::value || WIN) e = acc_row(r, 0) < ps.rows ? e : 0.f;
        pv[r] = e;
        dsv[r] = e * (dp[r] - ps.Dl[r]);
    };
    auto ppack = [&](int h, int w, const float (&pv)[16], const float (&dsv)[16]) {
        pk[h][w] = Ops::pack2(pv[8 * h + 2 * w], pv[8 * h + 2 * w + 1]);
        dsk[h][w] = Ops::pack2(dsv[8 * h + 2 * w], dsv[8 * h + 2 * w + 1]);
    };
    auto probs = [&](uint32_t b, int i0, const f32x16 &s, const f32x16 &dp, auto tail) {
        const PStat ps = pstats(b, i0);
        float pv[16], dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pelem(ps, r, s, dp, pv, dsv, tail);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w) ppack(h, w, pv, dsv);
    };
    auto grads = [&](uint32_t b) {
        u32x4 tg[2][DB], tq[2][DB];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const uint32_t co = (uint32_t)(kc * 16 * ROWB);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                tg[kc][db] = read_tr<DB>(smem + b + TILEB, rd_tr, db, co);
                tq[kc][db] = read_tr<DB>(smem + b, rd_tr, db, co);
            }
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dv[db] = Ops::mma(tg[kc][db], pk[kc], dv[db]);
                dk[db] = Ops::mma(tq[kc][db], dsk[kc], dk[db]);
            }
    };
    auto buf = [&](int t) { return (uint32_t)((t & (NBUF - 1)) * BUFB); };
    using no_tail = std::integral_constant<bool, false>;
    using with_tail = std::integral_constant<bool, true>;

    // One step: tile t+3 requested; S/dP of tile t+1 on the MFMA pipe while
    // the vector ALU forms the probabilities and dS of tile t (from the S/dP
    // of the previous step) and the transposing reads of the dV/dK operands
    // of tile t go out; then dV/dK of tile t.  Tile t+2 must have arrived by
    // the step's end.  The S/dP products are laid out one dimension chunk
    // at a time with their share of the elements and reads, each chunk
    // fenced from the next, so that the vector work fills the MFMA pipe's
    // time instead of following it.
    auto step = [&](int t) {
        const int i0 = i_begin + t * BQ;
        issue(i0 + 3 * BQ, buf(t + 3));
        const f32x16 sc = s, dpc = dp;
        const uint32_t bn = buf(t + 1), bc = buf(t);
        // the row statistics first: LDS reads complete in order, and the
        // first elements need them while the first products need only aq[0]
        const PStat ps = pstats(bc, i0);
        u32x4 aq[DC], ag[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            aq[dc] = *(const u32x4 *)(smem + bn + rd_row[dc]);
            ag[dc] = *(const u32x4 *)(smem + bn + TILEB + rd_row[dc]);
        }
        float pv[16], dsv[16];
        u32x4 tg[2][DB], tq[2][DB];
        constexpr int EPC = 16 / DC;          // elements per dimension chunk
        constexpr int RPC = 2 * DB / DC;      // operand pairs read per chunk (>= 1)
        static_assert(16 % DC == 0 && (2 * DB) % DC == 0 && RPC >= 1, "step split");
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            if (dc == 0) {
                s = Ops::mma(aq[0], kop[0], f32x16{});
                dp = Ops::mma(ag[0], vop[0], f32x16{});
            } else {
                s = Ops::mma(aq[dc], kop[dc], s);
                dp = Ops::mma(ag[dc], vop[dc], dp);
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) pelem(ps, dc * EPC + e, sc, dpc, pv, dsv, no_tail());
#pragma unroll
            for (int e = 0; e < EPC; e += 2) {
                const int r = dc * EPC + e;   // elements r, r+1 complete a pair
                ppack(r >> 3, (r & 7) >> 1, pv, dsv);
            }
#pragma unroll
            for (int x = 0; x < RPC; ++x) {
                const int idx = dc * RPC + x, kc = idx / DB, db = idx % DB;
                const uint32_t co = (uint32_t)(kc * 16 * ROWB);
                tg[kc][db] = read_tr<DB>(smem + bc + TILEB, rd_tr, db, co);
                tq[kc][db] = read_tr<DB>(smem + bc, rd_tr, db, co);
            }
#if BWD_KV_SCHED
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dv[db] = Ops::mma(tg[kc][db], pk[kc], dv[db]);
                dk[db] = Ops::mma(tq[kc][db], dsk[kc], dk[db]);
            }
        wait_vmcnt<LPI>();
        __syncthreads();
    };

    // The same step for two waves per SIMD (D = 64), where the partner wave
    // hides what one wave leaves idle: tile t+3 requested, S/dP of tile t+1,
    // dV/dK of tile t with the probabilities of tile t+1 between its
    // products (pinned with sched_group_barrier).
    auto step2 = [&](int t, auto tail) {
        const int i0 = i_begin + t * BQ;
        issue(i0 + 3 * BQ, buf(t + 3));
        sdp(buf(t + 1));
        grads(buf(t));
        probs(buf(t + 1), i0 + BQ, s, dp, tail);
#if BWD_KV_SCHED
        // the loads first; the S/dP operands; the S/dP products with the
        // transposing reads of the dV/dK operands between them; the dV/dK
        // products with the probabilities of tile t+1 between them
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DC, 0);        // DS read
#pragma unroll
        for (int n = 0; n < 2 * DC; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB / DC + 1, 0);
        }
#pragma unroll
        for (int n = 0; n < 4 * DB; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (n >= 2) __builtin_amdgcn_sched_group_barrier(0x002, BWD_KV_VPER, 0);  // VALU
        }
#endif
        wait_vmcnt<LPI>();
        __syncthreads();
    };

    if (ntiles > 0) {
        // tiles 0, 1, 2 (past the end: clamped rows, never used)
        issue(i_begin, buf(0));
        issue(i_begin + BQ, buf(1));
        issue(i_begin + 2 * BQ, buf(2));
        wait_vmcnt<LPI>();
        __syncthreads();
        sdp(buf(0));
        int t = 0;
        if constexpr (OCC == 1) {
            for (; t + 1 < ntiles; ++t) step(t);
            probs(buf(t), i_begin + t * BQ, s, dp, with_tail());
        } else {
            probs(buf(0), i_begin, s, dp, with_tail());
            for (; t + 2 < ntiles; ++t) step2(t, no_tail());
            if (t + 1 < ntiles) step2(t++, with_tail());
        }
        grads(buf(t));
    }
    wait_vmcnt<0>();

    // dK and dV as whole rows through the LDS, free once every wave is past
    // its last step: each wave uses its own 2 x 32 rows
    __syncthreads();
    {
        const uint32_t st = smem_base + (uint32_t)(wave * 2 * 32 * ROWB);
        const int nk = min(32, Lk - kw);
        store_rows_staged<Ops, D>(st, dk, p.scale, p.dk + dk_b + (int64_t)kw * dk_sl, dk_sl, nk,
                                  lane);
        store_rows_staged<Ops, D>(st + (uint32_t)(32 * ROWB), dv, 1.f,
                                  p.dv + dv_b + (int64_t)kw * dv_sl, dv_sl, nk, lane);
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per NW * 32 query rows, 32 per wave; key tiles of 64.
// ---------------------------------------------------------------------------
template <typename Ops, int D, bool CAUSAL, int OCC, int NW, bool GEN = false, bool WIN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_bwd_dq_mfma_kernel(BwdParams p)
{
    constexpr int BM = NW * 32;          // query rows per workgroup
    constexpr int BN = 64;               // keys per tile
    constexpr int KB = BN / 32, KC = BN / 16;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = BN * ROWB;
    constexpr int NLD = BN * CH / (NW * 64);
    constexpr int BUFB = 2 * TILEB;
    static_assert(NLD >= 1 && BN * CH % (NW * 64) == 0, "tile split");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUFB];
    static_assert(NW * 32 * ROWB <= 2 * BUFB, "dQ staging fits the LDS");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    int bh, qt;
    decompose(blockIdx.x, gridDim.x, p.BH, p.nt, CAUSAL, false, bh, qt);
    const int Lq = p.Lq, Lk = p.Lk;
    const int q_first = qt * BM;
    const int qw = q_first + wave * 32;
    const int qrow = qw + l32;
    const bool row_ok = qrow < Lq;

    int64_t q_b, g_b, k_b, v_b, dq_b;
    int q_sl, g_sl, k_sl, v_sl, dq_sl;
    tensor_at<GEN, D>(p, 0, bh, Lq, q_b, q_sl);
    tensor_at<GEN, D>(p, 4, bh, Lq, g_b, g_sl);
    tensor_at<GEN, D>(p, 1, bh, Lk, k_b, k_sl);
    tensor_at<GEN, D>(p, 2, bh, Lk, v_b, v_sl);
    tensor_at<GEN, D>(p, 5, bh, Lq, dq_b, dq_sl);
    const uint16_t *kh = p.k + k_b;
    const uint16_t *vh = p.v + v_b;

    // Q^T and dO^T operands (B of S^T = K Q^T and dP^T = V dO^T)
    u32x4 qop[DC], gop[DC];
    {
        const uint16_t *qr = p.q + q_b + (int64_t)qrow * q_sl + 8 * hi;
        const uint16_t *gr = p.dout + g_b + (int64_t)qrow * g_sl + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            qop[dc] = row_ok ? *(const u32x4 *)(qr + dc * 16) : u32x4{0u, 0u, 0u, 0u};
            gop[dc] = row_ok ? *(const u32x4 *)(gr + dc * 16) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const float lse2 = row_ok ? p.lse[(int64_t)bh * Lq + qrow] * kLog2e : INFINITY;
    const float dl = row_ok ? p.delta[(int64_t)bh * Lq + qrow] : 0.f;
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

    // Direct loads, as in the dK/dV kernel: load n of a wave fills LDS chunk
    // positions (n*NW + wave)*64 + lane of a tile.
    int dm_row[NLD];
    uint32_t dm_col[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int pos = (n * NW + wave) * 64 + lane;
        const int row = pos / CH, phys = pos % CH;
        dm_row[n] = row;
        dm_col[n] = (uint32_t)(((phys ^ swz<D>(row)) * 8));
    }
    const uint32_t smem_base = lds_addr(smem);
    uint32_t rd_row[DC];
    {
        const int row = swap_bits23(l32);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            rd_row[dc] = (uint32_t)(row * ROWB + (((2 * dc + hi) ^ swz<D>(row)) * 16));
    }
    uint32_t rd_tr[DB][2];
    tr_offsets<D, DB>(lane, rd_tr);

    // keys [kv_begin, kv_end) are visible to some row of the block
    int kv_begin = 0;
    int kv_end = CAUSAL ? min(Lk, q_first + BM) : Lk;
    if constexpr (WIN) {
        if (p.wl >= 0) kv_begin = max(0, q_first - p.wl);
        if (p.wr >= 0) kv_end = min(kv_end, q_first + BM + p.wr);
    }
    const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + BN - 1) / BN : 0;

    // Keys past the end fetch the last key (valid memory); their
    // probabilities are masked to zero.
    auto issue = [&](int k0, uint32_t b) {
        const uint32_t wb = uniform(smem_base + b + (uint32_t)(wave * 1024));
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int64_t row = min(k0 + dm_row[n], Lk - 1);
            dma_16B(kh + row * k_sl + dm_col[n], wb + (uint32_t)(n * NW * 1024));
            dma_16B(vh + row * v_sl + dm_col[n], wb + TILEB + (uint32_t)(n * NW * 1024));
        }
    };

    if (ntiles > 0) {
        issue(kv_begin, 0);
        wait_vmcnt<0>();
        __syncthreads();
    }
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = kv_begin + t * BN;
        const uint8_t *cur = smem + (t & 1) * BUFB;
        const bool more = t + 1 < ntiles;
        if (more) issue(k0 + BN, (uint32_t)(((t + 1) & 1) * BUFB));
        if (!CAUSAL || k0 <= qw + 31) {
            const uint8_t *kt = cur, *vt = cur + TILEB;
            // mask: keys past the diagonal (causal) or past the end
            bool need_mask = (CAUSAL && k0 + BN - 1 > qw) || k0 + BN > Lk;
            if constexpr (WIN)
                need_mask = need_mask || (p.wr >= 0 && k0 + BN - 1 > qw + p.wr) ||
                            (p.wl >= 0 && k0 < qw + 31 - p.wl);
            u32x4 dsk[KC];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 s, dp;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] = 0.f;
                    dp[i] = 0.f;
                }
                const uint32_t bo = (uint32_t)(kb * 32 * ROWB);
#pragma unroll
                for (int dc = 0; dc < DC; ++dc) {
                    s = Ops::mma(*(const u32x4 *)(kt + bo + rd_row[dc]), qop[dc], s);
                    dp = Ops::mma(*(const u32x4 *)(vt + bo + rd_row[dc]), gop[dc], dp);
                }
                // exponent arguments; masked ones become -inf (probability
                // 0, for any scale including 0).  Only tiles that cross the
                // diagonal, the window or the end of the keys take the mask
                // block (a separate block: inside the element loop the
                // compiler turned the uniform test into selects on every tile)
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], p.c, -lse2);
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = k0 + kb * 32 + acc_row(r, hi);
                        bool keep = j < Lk && (!CAUSAL || j <= qrow);
                        if constexpr (WIN)
                            keep = keep && (p.wr < 0 || j <= qrow + p.wr) &&
                                   (p.wl < 0 || j >= qrow - p.wl);
                        x[r] = keep ? x[r] : -INFINITY;
                    }
                }
                float dsv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] = exp2_fast(x[r]) * (dp[r] - dl);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        dsk[2 * kb + h][w] =
                            Ops::pack2(dsv[8 * h + 2 * w], dsv[8 * h + 2 * w + 1]);
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const uint32_t co = (uint32_t)(kc * 16 * ROWB);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dq[db] = Ops::mma(read_tr<DB>(kt, rd_tr, db, co), dsk[kc], dq[db]);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
    }

    // dQ as whole rows through the LDS (every tile ends with a barrier, so
    // no wave reads it any more): 32 rows per wave
    store_rows_staged<Ops, D>(smem_base + (uint32_t)(wave * 32 * ROWB), dq, p.scale,
                              p.dq + dq_b + (int64_t)qw * dq_sl, dq_sl, min(32, Lq - qw), lane);
}

template <typename Ops, int D, bool CAUSAL, bool GEN, bool WIN>
hipError_t launch_t(const BwdArgs &a)
{
    BwdParams p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.dout = static_cast<const uint16_t *>(a.dout);
    p.lse = a.lse;
    p.delta = a.delta;
    p.dq = static_cast<uint16_t *>(a.dq);
    p.dk = static_cast<uint16_t *>(a.dk);
    p.dv = static_cast<uint16_t *>(a.dv);
    p.BH = (int)(a.B * a.H);
    p.Lq = (int)a.Lq;
    p.Lk = (int)a.Lk;
    p.scale = a.scale;
    p.c = a.scale * kLog2e;
    p.H = (int)a.H;
    p.wl = a.wl;
    p.wr = a.wr;
    for (int t = 0; t < 8; ++t)
        for (int i = 0; i < 3; ++i) p.st[t][i] = a.st[t][i];
    constexpr int BLK = (kThreads / 64) * 32;
    p.nt = (int)((a.Lk + BLK - 1) / BLK);
    hipLaunchKernelGGL((fa_bwd_dkdv_mfma_kernel<Ops, D, CAUSAL, D == 64 ? BWD_KV_OCC64 : BWD_KV_OCC128, GEN, WIN>),
                       dim3((unsigned)(p.BH * p.nt)), dim3(kThreads), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int NWQ = D == 64 ? BWD_Q_NW64 : BWD_Q_NW128;
    p.nt = (int)((a.Lq + NWQ * 32 - 1) / (NWQ * 32));
    hipLaunchKernelGGL((fa_bwd_dq_mfma_kernel<Ops, D, CAUSAL, D == 64 ? BWD_Q_OCC64 : BWD_Q_OCC128, NWQ, GEN, WIN>),
                       dim3((unsigned)(p.BH * p.nt)), dim3(NWQ * 64), 0, a.stream, p);
    return hipGetLastError();
}

template <typename Ops, bool GEN, bool WIN>
hipError_t launch_gen(const BwdArgs &a)
{
    if (a.D == 64)
        return a.causal ? launch_t<Ops, 64, true, GEN, WIN>(a) : launch_t<Ops, 64, false, GEN, WIN>(a);
    return a.causal ? launch_t<Ops, 128, true, GEN, WIN>(a) : launch_t<Ops, 128, false, GEN, WIN>(a);
}

// contiguous and unwindowed: compile-time strides, no window code; strided
// without a window; strided with a window
template <typename Ops>
hipError_t launch_ops(const BwdArgs &a)
{
    if (!a.general) return launch_gen<Ops, false, false>(a);
    if (a.wl < 0 && a.wr < 0) return launch_gen<Ops, true, false>(a);
    return launch_gen<Ops, true, true>(a);
}

}  // namespace

bool bwd_mfma_supported(const BwdArgs &a)
{
    return (a.dtype == 1 || a.dtype == 2) && (a.D == 64 || a.D == 128);
}

hipError_t bwd_mfma_launch(const BwdArgs &a)
{
    return a.dtype == 1 ? launch_ops<F16Ops>(a) : launch_ops<Bf16Ops>(a);
}

const char *bwd_mfma_kernel_name(const BwdArgs &a)
{
    static const char *names[2][2][2] = {
        {{"fa_bwd_mfma_f16_d64", "fa_bwd_mfma_f16_d64_causal"},
         {"fa_bwd_mfma_f16_d128", "fa_bwd_mfma_f16_d128_causal"}},
        {{"fa_bwd_mfma_bf16_d64", "fa_bwd_mfma_bf16_d64_causal"},
         {"fa_bwd_mfma_bf16_d128", "fa_bwd_mfma_bf16_d128_causal"}},
    };
    return names[a.dtype == 2][a.D == 128][a.causal ? 1 : 0];
}

}  // namespace fa
