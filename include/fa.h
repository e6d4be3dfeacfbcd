/*
 * fa.h -- C ABI of libfa.so: the exact, IO-aware attention forward on MI355X
 * (gfx950).
 *
 * Operation.  For every batch b, query head h and query row i:
 *     s_ij  = scale * sum_x q[b,i,h,x] * k[b,j,hk,x]     for visible keys j
 *     o[b,i,h,:] = sum_j softmax_j(s_i.) * v[b,j,hk,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 * with hk = h / (Hq / Hkv).  This is standard attention for each head
 * ("[Attention优化] 从Online-Softmax到FlashAttention V1/V2/V3", section 0x01,
 * with the scale the page leaves out put back), multi-query / grouped-query
 * attention by indexing the shared key/value head (same page, section 0x09),
 * and the per-row statistics the forward keeps for the backward pass
 * ("FlashAttention：IO 感知的精确注意力", section 6), returned as the natural
 * log-sum-exp m + ln(l).  The result is exact up to floating-point rounding
 * (same page, section 5.1): tiles of Q, K and V are merged with the
 * online-softmax recurrence, and the N x N score matrix never reaches memory.
 *
 * Causal mask (causal != 0), aligned to the bottom-right corner of the
 * score matrix as the first page's section 0x09 states for unequal lengths:
 * key j is visible to query i iff j <= i + (Nk - Nq).  With one length N
 * (fa_fwd, fa_fwd_f32) this is j <= i.  A query row that sees no key (only
 * possible when Nq > Nk) gets an all-zero output row, as that section says,
 * and lse = -inf.
 *
 * Layout.  All tensors are dense, contiguous, row-major (C order):
 *     q, o : [B][Nq][Hq][d]     k, v : [B][Nk][Hkv][d]     lse : [B][Hq][Nq]
 * Element (b,n,h,x) of q is at ((b*Nq + n)*Hq + h)*d + x.  fa_fwd and
 * fa_fwd_f32 take one length N = Nq = Nk.
 *
 * Ownership.  Every pointer is a DEVICE pointer owned by the caller.  The
 * library allocates nothing, keeps no state between calls and never
 * synchronises.  It reads q, k, v, writes every element of o and lse (and,
 * for a split forward, the caller's workspace), and writes nothing else.
 * Calls are re-entrant; calls that share a workspace must not overlap in
 * time (enqueue them on one stream).
 *
 * Errors.  Arguments are validated before any HIP call; on a validation error
 * the function returns a nonzero status and enqueues nothing.  On success the
 * work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 * function returns FA_OK without waiting.  FA_ERR_LAUNCH reports a failure
 * that the HIP runtime returned for the launch.  (HIP's last-error state is
 * cleared right before the launches, so that an earlier failure of another
 * HIP call in the thread, already returned to its own caller, is not
 * reported as this launch's.)  Faults during execution
 * surface at the caller's next synchronisation.  Non-finite input values
 * propagate into the results (no check is made).  No C++ exception crosses
 * this interface.
 *
 * Limits.  d in {64, 128, 256} for the bf16 forward (fa_fwd, fa_fwd_splitkv),
 * {64, 128} for the fp32 forward and the backward, 128 for fa_fwd_fp8;
 * B, Hq, Hkv, Nq, Nk >= 1; Hq % Hkv == 0;
 * (Nq + 256) * Hq * d < 2^29 and (Nk + 256) * Hkv * d < 2^29 (elements per
 * batch entry of one tensor); B * Hq * ceil(Nq / 128) * splits < 2^31.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,     /* a required pointer is NULL                          */
    FA_ERR_SHAPE = 2,    /* B, Hq, Hkv or N < 1, or a size limit exceeded        */
    FA_ERR_HEADS = 3,    /* Hq is not a multiple of Hkv                          */
    FA_ERR_HEADDIM = 4,  /* d not supported by this entry point (see Limits)      */
    FA_ERR_ALIGN = 5,    /* q, k, v or o not 16-byte aligned; lse not 4-byte     */
    FA_ERR_SCALE = 6,    /* scale not finite, or |scale|*log2(e) not a normal float (scale 0 is allowed) */
    FA_ERR_ALIAS = 7,    /* o or lse overlaps q, k, v or each other              */
    FA_ERR_LAUNCH = 8,   /* the HIP runtime reported an error for the launch     */
    FA_ERR_SPLITS = 9,   /* num_splits outside 0..256                            */
    FA_ERR_WORKSPACE = 10, /* split forward: workspace NULL, too small or not 16-byte aligned */
    FA_ERR_SCRATCH = 11  /* fa_fwd_splitkv_static: the split needs more than FA_STATIC_SCRATCH_BYTES */
} fa_status;

/*
 * fa_fwd -- bf16 inputs and output, fp32 accumulation and statistics.
 *   q, k, v : bf16 (raw 16-bit bfloat16) device arrays in the layout above.
 *   o       : bf16 output, same layout as q, rounded to nearest even.
 *   lse     : fp32 output [B][Hq][N].
 *   scale   : a finite float, applied to q.k before the mask; 0 is allowed,
 *             otherwise |scale|*log2(e) must be a normal float.
 *   causal  : 0 = every key visible, nonzero = key j visible iff j <= i.
 *   (Also reachable as fa_fwd_splitkv with Nq = Nk = N and num_splits = 1.)
 *   stream  : hipStream_t to enqueue on (NULL = null stream).
 * Returns an fa_status value.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal,
           void *stream);

/*
 * fa_fwd_f32 -- the same operation with fp32 inputs and output (fp32
 * arithmetic throughout).  Same arguments, layouts, limits and errors.
 */
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o,
               float *lse, int B, int Hq, int Hkv, int N, int d, float scale,
               int causal, void *stream);

/*
 * fa_fwd_splitkv -- bf16 attention with separate query and key lengths, the
 * key sequence optionally split into ranges that run in parallel.
 *
 * The keys are cut into num_splits contiguous ranges (multiples of 64 keys,
 * none empty; fewer ranges are used when Nk is short).  Every range is
 * processed by its own workgroups, which store for each query row the
 * softmax over that range applied to its V rows (fp32) and the range's
 * log-sum-exp; a second kernel then merges the ranges with the online-softmax
 * rescaling ("FlashAttention：IO 感知的精确注意力", section 5; its section 12.1
 * describes this split for decoding, where one query row meets a long key
 * sequence and batch x heads alone cannot fill the GPU).  The result is the
 * same operation as fa_fwd, up to rounding.
 *   q, o      : bf16 [B][Nq][Hq][d];  k, v : bf16 [B][Nk][Hkv][d];
 *   lse       : fp32 [B][Hq][Nq].
 *   Nq, Nk    : query and key lengths (causal alignment as above).
 *   num_splits: 1 = no split (workspace unused, may be NULL); 2..256 = at
 *               most that many ranges; 0 = chosen by fa_splitkv_num_splits.
 *   workspace : device memory of at least fa_splitkv_workspace_size(...)
 *               bytes, 16-byte aligned, owned by the caller; its contents on
 *               entry do not matter and are overwritten.
 * Other arguments, errors and limits as for fa_fwd.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                   int causal, int num_splits, void *workspace,
                   size_t workspace_bytes, void *stream);

/* fa_fwd_splitkv with fp32 inputs, output and arithmetic. */
int fa_fwd_splitkv_f32(const float *q, const float *k, const float *v, float *o,
                       float *lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       float scale, int causal, int num_splits, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * fa_fwd_splitkv_static -- fa_fwd_splitkv for callers that cannot allocate
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments and kernels, but the
 * per-range partial results go to a static device array of the library,
 * FA_STATIC_SCRATCH_BYTES long, instead of a caller workspace.  The call
 * allocates nothing.  Each GPU holds its own array until the process ends;
 * its device address is looked up (hipGetSymbolAddress) on the first call
 * on that device.  Every call on one GPU shares that array, so calls that
 * overlap in time on one GPU race: enqueue them on one stream.  Returns
 * FA_ERR_SCRATCH, before any HIP call, when the split needs more scratch
 * than the array holds (fa_splitkv_workspace_size tells how much it needs);
 * FA_ERR_LAUNCH if the array's address cannot be obtained.  Other errors as
 * fa_fwd_splitkv.
 */
#define FA_STATIC_SCRATCH_BYTES (32u << 20)
int fa_fwd_splitkv_static(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                          int causal, int num_splits, void *stream);

/*
 * Number of key ranges fa_fwd_splitkv uses for these arguments (num_splits
 * as passed to it; 0 picks enough ranges for about two workgroups per
 * compute unit, each range at least 256 keys).  Returns a value >= 1, or
 * minus an fa_status for invalid arguments.
 */
int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/*
 * Workspace bytes fa_fwd_splitkv needs for these arguments:
 * ranges * B * Hq * Nq * (d + 1) * 4 (partial outputs, then partial
 * log-sum-exps), or 0 when one range is used or the arguments are invalid.
 */
size_t fa_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/*
 * fa_fwd_blocksparse -- fa_fwd restricted to the blocks a block mask keeps:
 * the block-sparse variant of the first page's section 0x04, where blocks
 * of the score matrix that a sparsity pattern marks are skipped entirely.
 *   block_mask : device bytes [Hq][ceil(N/128)][ceil(N/64)]; entry [h][a][c]
 *                nonzero keeps keys 64c .. 64c+63 for query rows
 *                128a .. 128a+127 of head h (together with the causal rule).
 * Each row's softmax runs over its kept keys alone; a row that keeps none
 * gets O = 0 and lse = -inf.  Skipped blocks cost no memory traffic and no
 * arithmetic.  bf16 as fa_fwd; d in {64, 128, 256}; N <= 65536.  Other
 * arguments, errors and limits as for fa_fwd; FA_ERR_NULL for a NULL mask.
 */
int fa_fwd_blocksparse(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       const unsigned char *block_mask, void *stream);

/*
 * fa_fwd_fp8 -- the forward with fp8 inputs: the low-precision path of the
 * second page's section 10 (FlashAttention-3 FP8) with per-block scales
 * (section 12.2), one block per (batch, head).
 *   q, k, v   : OCP e4m3 (E4M3FN) codes, one byte per element, laid out as
 *               fa_fwd's q, k, v.  The real inputs are code * descale:
 *   q_descale : fp32 [B][Hq], k_descale and v_descale : fp32 [B][Hkv] (device).
 *   o         : bf16 [B][N][Hq][d], round to nearest even.
 *   lse       : fp32 [B][Hq][N], of the real scaled scores.
 * The scores come from the fp8 matrix cores (exact products, fp32 sums).  The
 * probabilities are quantised to e4m3 for the P V product (relative error at
 * most 2^-4 each, against a running maximum so that none saturates), and O
 * is normalised by the sum of the quantised values, so every output row is a
 * convex combination of V rows with weights within 2^-4 of the exact ones.
 * d must be 128.  Other arguments, errors and limits as for fa_fwd; the
 * descale pointers must be non-NULL and 4-byte aligned.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, const float *q_descale,
               const float *k_descale, const float *v_descale, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream);

/*
 * fa_fwd_fp8_block -- the fp8 forward with per-block scales: the block
 * quantisation that the second page ("FlashAttention：IO 感知的精确注意力",
 * section 10, FlashAttention-3's FP8 path; section 12.2) recommends over one
 * scale per tensor.  A block is 64 consecutive rows (sequence positions) of
 * one head, and its scale a power of two:
 *   q, k, v   : e4m3 codes laid out as fa_fwd_fp8's (one byte each);
 *   q_exp     : int8 [B][Hq][ceil(N/64)], k_exp and v_exp : int8
 *               [B][Hkv][ceil(N/64)] (device); the real input of row n of
 *               head h is code * 2^exp[b][h][n / 64] (fa_quantize_fp8 writes
 *               such codes and exponents).
 * The scales are applied exactly by the matrix cores' block-scaled fp8
 * products.  Output, probabilities, normalisation, error bound and
 * arguments otherwise as fa_fwd_fp8 (d must be 128; the exponent pointers
 * must be non-NULL and must not overlap o or lse).
 */
int fa_fwd_fp8_block(const void *q, const void *k, const void *v, const signed char *q_exp,
                     const signed char *k_exp, const signed char *v_exp, void *o, float *lse,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream);

/*
 * fa_quantize_fp8 -- block-scaled e4m3 quantisation of a bf16 tensor for
 * fa_fwd_fp8_block, with optional incoherent processing (the rotation that
 * spreads outlier coordinates before quantisation, same page, section 10).
 *   x      : bf16 [B][N][H][d] (device), d = 128;
 *   signs  : NULL, or int8 [d] of +1 / -1 (device, 8-byte aligned): each row
 *            is first rotated, y = (x * signs) H, H the d x d
 *            Sylvester-Hadamard matrix (H[i][j] = (-1)^popcount(i & j)),
 *            computed in fp32 by the radix-2 butterfly network in stage
 *            order h = 1, 2, 4, ..., d/2.  Rotating both q and k with the
 *            same signs multiplies every score by d exactly, so the
 *            attention takes scale / d; v is not rotated.
 *   codes  : e4m3 [B][N][H][d] (device, 8-byte aligned), written;
 *   exps   : int8 [B][H][ceil(N/64)] (device), written: for each block of
 *            64 rows of a head, the smallest e with max|y| / 2^e <= 448 (the
 *            largest e4m3 value), -127 for an all-zero block; the codes are
 *            the e4m3 values nearest to y / 2^e, ties to even.
 * Rows whose |x| * d overflows fp32 are not supported (no check is made).
 * Returns FA_ERR_NULL, FA_ERR_SHAPE (sizes as fa_fwd's limits),
 * FA_ERR_HEADDIM (d != 128), FA_ERR_ALIGN (x 16-byte, codes and signs
 * 8-byte), FA_ERR_ALIAS (outputs overlapping inputs or each other) before
 * any HIP call, else FA_OK or FA_ERR_LAUNCH.
 */
int fa_quantize_fp8(const void *x, void *codes, signed char *exps, int B, int N, int H, int d,
                    const signed char *signs, void *stream);

/*
 * fa_bwd -- gradients of the bf16 forward (fa_fwd / fa_fwd_splitkv) for an
 * upstream gradient dout = dL/do.
 *
 *   dv = P^T dout,  dq = scale * dS k,  dk = scale * dS^T q,
 *   dS = P o (dout v^T - delta),  delta_i = sum_x dout[i,x] * o[i,x],
 * with P = exp(scale q k^T - lse) recomputed from the forward's lse (zero
 * where masked) rather than stored: the backward of the first page's
 * sections 0x04 and 0x05 and of the second page's section 6
 * ("FlashAttention：IO 感知的精确注意力").  For grouped-query attention dk and
 * dv of a key/value head are summed over the query heads that read it.
 *   q, o, dout, dq : bf16 [B][Nq][Hq][d];   k, v, dk, dv : bf16 [B][Nk][Hkv][d];
 *   lse            : fp32 [B][Hq][Nq], as fa_fwd wrote it (rows without keys
 *                    hold -inf and get zero gradients);
 *   o              : the forward's output for the same q, k, v, scale, causal;
 *   scale, causal  : as passed to the forward;
 *   workspace      : at least fa_bwd_workspace_size(B, Hq, Nq) bytes of device
 *                    memory, 4-byte aligned, owned by the caller; overwritten
 *                    (it receives delta and lse * log2(e) per row).
 * dq, dk, dv are fully written, rounded to nearest even.  Two kernels are
 * enqueued on `stream`: dq (query-block outer, also writing delta) and then
 * dk, dv (key-block outer).  The result is deterministic (no atomics).
 * Errors and limits as for fa_fwd_splitkv, plus FA_ERR_WORKSPACE for a
 * missing or short workspace; every output must be 16-byte aligned and
 * overlap no input, no other output and not the workspace.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, int B, int Hq, int Hkv,
           int Nq, int Nk, int d, float scale, int causal, void *workspace,
           size_t workspace_bytes, void *stream);

/* Workspace bytes fa_bwd needs: 2 * B * Hq * Nq * 4 (the rows' delta and
 * lse in base 2; 0 for invalid sizes). */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq);

/* Human-readable text for an fa_status value (static storage, never NULL). */
const char *fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/* LDS stages of the kernels this library was built with: 2 in the normal
 * build, where the next tile (K/V in the forward kernels and the dQ kernel,
 * Q/dO in the dK/dV kernel) streams into one stage while the other is read;
 * 1 in the debug build (libfa_single_stage.so), which loads each tile only
 * after every read of the one stage has ended; 0 if the kernel sources were
 * built inconsistently.  The debug build exists to check the normal build's
 * wait and barrier placement: its outputs must be equal bit for bit.  Covers
 * the bf16, fp8 and fp32 forward kernels and the backward; the decoding
 * kernel keeps one stage in both builds.  No error case. */
int fa_lds_stages(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
