// fa_internal.h -- declarations shared by the library's host and kernel
// sources.  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Arguments of one forward call after validation.  Strides are in elements
// (batch, head, row) per tensor, the head dimension is contiguous; fa_fwd
// fills in the contiguous [B, H, L, D] strides.  wl / wr: local window
// bounds (query i keeps key j when i - wl <= j <= i + wr), -1 = no bound.
// general: strides are not the contiguous ones or a window is set.
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t B, H, Lq, Lk, D;
    int causal;
    float scale;
    int dtype;
    hipStream_t stream;
    int64_t qs[3], ks[3], vs[3], os[3];
    int wl, wr;
    bool general;
};

// Tile shape of the MFMA kernel: NW waves per workgroup, each wave owning
// QB blocks of 32 queries (so BM = NW * QB * 32 query rows per workgroup),
// BN keys per K/V tile, OCC waves per SIMD the register budget is cut for,
// and the K/V pipe: 0 stages tiles through VGPRs with a transposing V store,
// one tile per step; 2 loads tiles straight into LDS, reads V^T with
// transposing LDS reads and software-pipelines the QK^T of the next tile
// under the softmax of this one; 3 (8x1x64x2 only) is the ping-pong kernel,
// in which the two waves of each SIMD alternate MFMA and softmax phases.
struct MfmaTile {
    int nw, qb, bn, occ, pipe;
};

// MFMA kernel: fp16/bf16 I/O, D in {64, 128}, scale > 0.
bool mfma_supported(const FwdArgs &a);
MfmaTile mfma_choose_tile(const FwdArgs &a);
const char *mfma_kernel_name(const FwdArgs &a, const MfmaTile &t);
hipError_t mfma_launch(const FwdArgs &a, const MfmaTile &t);
// Strided / windowed calls: the software-pipelined kernel with runtime
// strides and window (8 waves when the grid is large, else 4).
const char *mfma_general_kernel_name(const FwdArgs &a);
hipError_t mfma_launch_general(const FwdArgs &a);

// Vector-ALU kernel: any I/O type, D in {64, 128}, any finite scale.
const char *valu_kernel_name(const FwdArgs &a);
hipError_t valu_launch(const FwdArgs &a);

// Arguments of one backward call after validation.  Element strides
// (batch, head, row) of q, k, v, o, dout, dq, dk, dv in that order; fa_bwd
// fills in the contiguous ones.  wl / wr and general as for FwdArgs.
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *delta;
    int64_t B, H, Lq, Lk, D;
    int causal;
    float scale;
    int dtype;
    hipStream_t stream;
    int64_t st[8][3];
    int wl, wr;
    bool general;
};
enum { kQ = 0, kK, kV, kO, kDout, kDq, kDk, kDv };

// delta_i = dO_i . O_i into a.delta (any I/O type).
hipError_t bwd_delta_launch(const BwdArgs &a);

// MFMA backward (dK/dV kernel, then dQ kernel): fp16/bf16 I/O, D in {64, 128}.
bool bwd_mfma_supported(const BwdArgs &a);
const char *bwd_mfma_kernel_name(const BwdArgs &a);
hipError_t bwd_mfma_launch(const BwdArgs &a);

// Vector-ALU backward (dK, dV, then dQ): any I/O type, D in {64, 128}.
const char *bwd_valu_kernel_name(const BwdArgs &a);
hipError_t bwd_valu_launch(const BwdArgs &a);

}  // namespace fa
