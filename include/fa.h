/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward library.
 *
 * The library (libfa.so) computes scaled dot-product attention
 *
 *     O   = softmax(scale * Q K^T  [+ causal mask]) V
 *     LSE = log(sum_j exp(scale * q_i . k_j))      (natural log, visible j)
 *
 * with an online softmax over streamed K/V tiles, so the Lq x Lk score matrix
 * never reaches device memory.  Definitions: "Triton Ascend Attention",
 * section "standard attention computation flow" (scaled scores, row softmax,
 * weighted sum) and section "Flash Attention optimisation strategy / online
 * softmax"; the FlashAttention-2 forward article (wsisp.com): the host wrapper
 * (Q/K/V as [B, H, L, D] tensors, output allocated like Q, a [B, H, Lq] fp32
 * row statistic), the kernel epilogue (stores m + log(l)) and _attn_fwd_inner
 * (K/V streamed in blocks, causal predicate offs_m >= offs_n).
 *
 * All entry points are plain C; no C++ or framework types cross this line.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o (one type for all four). */
enum fa_dtype {
    FA_F32 = 0,  /* IEEE binary32 */
    FA_F16 = 1,  /* IEEE binary16 */
    FA_BF16 = 2  /* bfloat16 */
};

/* Return codes.  FA_OK is zero; every error is positive. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* B, H, Lq or Lk < 1, or a size past the limits */
    FA_ERR_HEAD_DIM = 3,  /* D is not 64 or 128 */
    FA_ERR_DTYPE = 4,     /* dtype is not one of enum fa_dtype */
    FA_ERR_SCALE = 5,     /* scale is NaN or infinite */
    FA_ERR_ALIGN = 6,     /* a tensor not 16-byte aligned, lse/delta not 4-byte */
    FA_ERR_ALIAS = 7,     /* an output overlaps an input or another output */
    FA_ERR_POINTER = 8,   /* a pointer is not device memory of this device */
    FA_ERR_LAUNCH = 9,    /* the HIP runtime rejected the kernel launch */
    FA_ERR_STRIDE = 10,   /* fa_fwd_ex: a stride is negative or too large, or o
                             is a view whose elements overlap */
    FA_ERR_SCRATCH = 11   /* fa_bwd_noalloc: B*H*Lq > FA_NOALLOC_MAX_ROWS */
};

/* Size limits checked by fa_fwd (FA_ERR_SHAPE past them). */
#define FA_MAX_SEQ  (1LL << 24)   /* Lq, Lk <= 16,777,216 */
#define FA_MAX_HEADS (1LL << 24)  /* B * H  <= 16,777,216 */

/*
 * fa_fwd -- attention forward on one GPU, enqueued on `stream`.
 *
 * q    [B, H, Lq, D]  device pointer, contiguous row-major (D fastest).
 * k    [B, H, Lk, D]  device pointer, contiguous row-major.
 * v    [B, H, Lk, D]  device pointer, contiguous row-major.
 * o    [B, H, Lq, D]  device pointer, written; same element type as q.
 * lse  [B, H, Lq]     device pointer to fp32, written at (b*H + h)*Lq + i;
 *                     may be NULL, then the row statistic is not stored.
 * B, H         batch and heads (the kernel grid runs over both, as in the
 *              article's launch grid of query blocks x batch*heads).
 * Lq, Lk       query and key lengths; independent (cross-attention).
 * D            head dimension, 64 or 128.
 * causal       nonzero: query i sees key j only when j <= i (diagonal kept,
 *              indices counted from the top-left corner, also when Lq != Lk).
 * scale        multiplies Q K^T; any finite value (the article's host wrapper
 *              passes 1/sqrt(D); the caller decides here).
 * dtype        enum fa_dtype of q, k, v, o.
 * stream       a hipStream_t; NULL is the null stream of the current device.
 *
 * Semantics: for each (b, h, i), with J_i the visible keys,
 *   o[b,h,i,:] = sum_{j in J_i} p_ij v[b,h,j,:],
 *   p_ij = exp(s_ij - m_i) / l_i,  s_ij = scale * q[b,h,i,:] . k[b,h,j,:],
 *   lse[b,h,i] = m_i + log(l_i).
 * bf16/fp16 inputs are multiplied exactly and accumulated in fp32; the
 * softmax runs in fp32; p is rounded to nearest-even into the I/O type for
 * the product with v, and o is divided by the sum of those rounded p (the
 * weights it was built from), then rounded to nearest-even into the I/O
 * type.  lse takes l from the fp32 sum of p for bf16, and from the sum of
 * the rounded p for fp16 (within 2^-10 of the fp32 sum: at most 9.8e-4 on
 * lse for rows up to 16384 keys).
 *
 * Ownership: the caller owns every buffer; the library allocates nothing,
 * keeps no state between calls and may be called from several threads.
 * o and lse must not overlap q, k, v or each other.
 *
 * Errors: every check runs on the host before anything is enqueued, in
 * this order: NULL pointers, sizes and limits, head dimension, dtype, scale,
 * alignment and overlaps use no HIP call; the last check, FA_ERR_POINTER,
 * asks the HIP runtime (hipGetDevice, hipPointerGetAttributes) whether each
 * pointer is device memory of the current device.  On an error nothing is
 * written and nothing is launched.  The launch itself is asynchronous: a
 * device fault appears at the caller's next synchronisation.
 * Returns FA_OK or an enum fa_status code.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
           int causal, float scale, int dtype, void *stream);

/*
 * fa_bwd -- gradients of the attention forward on one GPU, enqueued on
 * `stream`.
 *
 * The pages implement only the forward.  The FlashAttention-2 forward
 * article's host wrapper keeps Q, K, V, O and the row statistic for a
 * backward pass, its account of the IO-aware idea notes that a backward may
 * recompute the probabilities rather than store them, and its closing
 * remarks leave the backward as future work.  This entry point is the chain
 * rule through the forward's definition (see fa_fwd), with the probabilities
 * recomputed from lse; lse itself takes no gradient.  For each (b, h):
 *
 *   p_ij    = exp(s_ij - lse_i)   (s_ij as in fa_fwd; 0 for invisible keys)
 *   delta_i = dout_i . o_i
 *   ds_ij   = p_ij (dout_i . v_j - delta_i)
 *   dv_j    = sum_i p_ij dout_i
 *   dk_j    = scale * sum_i ds_ij q_i
 *   dq_i    = scale * sum_j ds_ij k_j
 *
 * q, k, v, causal, scale, dtype, B, H, Lq, Lk, D: exactly as passed to the
 *              fa_fwd call that produced o and lse.
 * o    [B, H, Lq, D]  device pointer, the forward output (I/O type).
 * lse  [B, H, Lq]     device pointer to fp32, the forward's row statistic.
 * dout [B, H, Lq, D]  device pointer, the incoming gradient of o.
 * dq   [B, H, Lq, D]  device pointer, written (I/O type).
 * dk   [B, H, Lk, D]  device pointer, written (I/O type).
 * dv   [B, H, Lk, D]  device pointer, written (I/O type).
 * delta [B, H, Lq]    device pointer to fp32 owned by the caller, written
 *              with delta_i (the library allocates nothing, so this per-row
 *              workspace is an argument; its contents are valid after the
 *              call completes).
 * All tensors contiguous row-major (D fastest), same element type.
 *
 * bf16/fp16 inputs: products exact, sums in fp32, probabilities and ds
 * rounded to the I/O type before they multiply tensors, gradients rounded to
 * nearest-even into the I/O type.  fp32 inputs: fp32 throughout.
 *
 * Ownership and errors as for fa_fwd: every check runs on the host before
 * anything is enqueued (FA_ERR_NULL for any NULL pointer, FA_ERR_ALIGN when a
 * tensor is not 16-byte or lse/delta not 4-byte aligned, FA_ERR_ALIAS when
 * dq, dk, dv or delta overlaps an input or another output); nothing is
 * written on an error.  Several kernels are enqueued in order on `stream`.
 * Deterministic: no atomics, the same inputs give the same bits.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const float *lse, const void *dout, void *dq, void *dk, void *dv,
           float *delta, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
           int64_t D, int causal, float scale, int dtype, void *stream);

/*
 * fa_fwd_ex -- the forward of fa_fwd on strided views and with an optional
 * local (sliding-window) mask, enqueued on `stream`.
 *
 * The FlashAttention-2 forward article's host wrapper hands the kernel the
 * batch, head, sequence and feature strides of Q, K, V and O, and the kernel
 * addresses every block with them (the wrapper and the kernel's offset
 * arithmetic).  Here the feature dimension must be contiguous (stride 1,
 * which the 16-byte vector loads need); the other three strides are free.
 * The article leaves other mask variants for later; the local window is the
 * common one: query i keeps key j only when i - window_left <= j and
 * j <= i + window_right.
 *
 * strides  12 int64 values, in elements: q (batch, head, row), then k, v,
 *          o in the same order.  Element (b, h, i, d) of q is at
 *          q + b*strides[0] + h*strides[1] + i*strides[2] + d.  For the
 *          [B, L, H, D] layout (sequence before heads) pass
 *          (L*H*D, D, H*D).  Every stride must be >= 0, at most 2^40, row
 *          strides at most 2^24, and a multiple of 8 elements (bf16/fp16) or
 *          4 (fp32) so rows stay 16-byte aligned; o must not map two elements
 *          to one address.  Inputs may overlap each other (packed QKV).
 * causal, window_left, window_right
 *          the keep rule is the conjunction of: (causal == 0 or j <= i),
 *          (window_left < 0 or j >= i - window_left),
 *          (window_right < 0 or j <= i + window_right).  A row that keeps no
 *          key gets o = 0 and lse = -inf.
 * lse      contiguous [B, H, Lq] fp32 as for fa_fwd, or NULL.
 * Other arguments, semantics, precision, ownership and errors as fa_fwd;
 * FA_ERR_STRIDE for invalid strides.  A call with the contiguous strides
 * and no window runs exactly fa_fwd.
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
              const int64_t *strides, int causal, int64_t window_left,
              int64_t window_right, float scale, int dtype, void *stream);

/*
 * fa_bwd_ex -- the gradients of fa_fwd_ex: fa_bwd on strided views and with
 * the same local window as the forward call that produced o and lse.
 *
 * strides  24 int64 values, in elements: (batch, head, row) of q, k, v, o,
 *          dout, dq, dk, dv, in that order; the same rules as fa_fwd_ex
 *          (feature dimension contiguous, strides >= 0 and 16-byte
 *          multiples, dq / dk / dv must not map two elements to one
 *          address).  lse and delta stay contiguous [B, H, Lq] fp32.
 * causal, window_left, window_right
 *          the keep rule of the forward (see fa_fwd_ex); gradients are zero
 *          for the pairs it drops.
 * Other arguments, semantics, precision, ownership and errors as fa_bwd.
 * A call with the contiguous strides and no window runs exactly fa_bwd.
 */
int fa_bwd_ex(const void *q, const void *k, const void *v, const void *o,
              const float *lse, const void *dout, void *dq, void *dk, void *dv,
              float *delta, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
              int64_t D, const int64_t *strides, int causal,
              int64_t window_left, int64_t window_right, float scale, int dtype,
              void *stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same gradients, kernels and precision as fa_bwd, but the
 * per-row statistic delta lives in a fixed scratch array inside the library
 * instead of a caller workspace, so there is no delta argument.  Nothing is
 * allocated: no hipMalloc, hipFree or allocating library call.
 *
 * Limit: B*H*Lq <= FA_NOALLOC_MAX_ROWS (2^21 rows, an 8 MiB fp32 array that
 * each GPU the library runs on holds until the process ends); larger calls
 * return FA_ERR_SCRATCH before anything is enqueued.
 * Sharing: every call on one GPU uses that GPU's one array, so calls that
 * overlap in time on one GPU (different streams or threads) race on it and
 * must be serialised by the caller.  Every call writes the rows it reads
 * before reading them, so nothing needs clearing between calls.
 * Arguments, ownership and the other errors as fa_bwd (contiguous tensors).
 */
#define FA_NOALLOC_MAX_ROWS (1LL << 21)
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const float *lse, const void *dout, void *dq, void *dk, void *dv,
                   int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                   int causal, float scale, int dtype, void *stream);

/* Static text for a status code ("unknown status" for anything else). */
const char *fa_status_string(int status);

/*
 * fa_kernel_name -- label of the kernel fa_fwd would launch for these
 * arguments (a static string), or NULL when fa_fwd would reject the shape,
 * head dimension, dtype or scale.  MFMA kernels are labelled
 * "fa_fwd_mfma_<bf16|f16>_d<D>[_causal]_<family><waves>w[<QB>q]_bn<keys>",
 * family ppp (persistent ping-pong), pp (ping-pong), pipe (software-
 * pipelined) or reg (register-staged, "_occ<waves per SIMD>" appended);
 * the vector-ALU kernel "fa_fwd_valu_<type>_d<D>[_causal]".  Host logic: it
 * launches and allocates nothing, but the choice of the persistent kernel
 * depends on the current device's compute-unit count (one HIP attribute
 * query; with no device that kernel is never named).  Used to label
 * measurements and to match profiler output.
 */
const char *fa_kernel_name(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                           int64_t D, int causal, float scale, int dtype);

/*
 * fa_bwd_kernel_name -- name of the gradient kernel (dk/dv) fa_bwd would
 * launch for these arguments, or NULL when fa_bwd would reject them.  Pure
 * host logic, like fa_kernel_name.
 */
const char *fa_bwd_kernel_name(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                               int64_t D, int causal, float scale, int dtype);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
