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
 * Causal mask (causal != 0): key j is visible to query i iff j <= i.  Query
 * and key sequences have the same length N, so the top-left and bottom-right
 * alignments of the first page's section 0x09 coincide and no row is empty.
 *
 * Layout.  All tensors are dense, contiguous, row-major (C order):
 *     q, o : [B][N][Hq][d]      k, v : [B][N][Hkv][d]      lse : [B][Hq][N]
 * Element (b,n,h,x) of q is at ((b*N + n)*Hq + h)*d + x.
 *
 * Ownership.  Every pointer is a DEVICE pointer owned by the caller.  The
 * library allocates nothing, keeps no state between calls and never
 * synchronises.  It reads q, k, v, writes every element of o and lse, and
 * writes nothing else.  Calls are re-entrant.
 *
 * Errors.  Arguments are validated before any HIP call; on a validation error
 * the function returns a nonzero status and enqueues nothing.  On success the
 * work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 * function returns FA_OK without waiting.  FA_ERR_LAUNCH reports a failure
 * that the HIP runtime returned for the launch.  Faults during execution
 * surface at the caller's next synchronisation.  Non-finite input values
 * propagate into the results (no check is made).  No C++ exception crosses
 * this interface.
 *
 * Limits.  d in {64, 128}; B, Hq, Hkv, N >= 1; Hq % Hkv == 0;
 * (N + 256) * max(Hq, Hkv) * d < 2^29 (elements per batch entry of one tensor);
 * B * Hq * ceil(N / 128) < 2^31.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,     /* a required pointer is NULL                          */
    FA_ERR_SHAPE = 2,    /* B, Hq, Hkv or N < 1, or a size limit exceeded        */
    FA_ERR_HEADS = 3,    /* Hq is not a multiple of Hkv                          */
    FA_ERR_HEADDIM = 4,  /* d is not 64 or 128                                   */
    FA_ERR_ALIGN = 5,    /* q, k, v or o not 16-byte aligned; lse not 4-byte     */
    FA_ERR_SCALE = 6,    /* scale not finite, or |scale|*log2(e) not a normal float (scale 0 is allowed) */
    FA_ERR_ALIAS = 7,    /* o or lse overlaps q, k, v or each other              */
    FA_ERR_LAUNCH = 8    /* the HIP runtime reported an error for the launch     */
} fa_status;

/*
 * fa_fwd -- bf16 inputs and output, fp32 accumulation and statistics.
 *   q, k, v : bf16 (raw 16-bit bfloat16) device arrays in the layout above.
 *   o       : bf16 output, same layout as q, rounded to nearest even.
 *   lse     : fp32 output [B][Hq][N].
 *   scale   : a finite float, applied to q.k before the mask; 0 is allowed,
 *             otherwise |scale|*log2(e) must be a normal float.
 *   causal  : 0 = every key visible, nonzero = key j visible iff j <= i.
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

/* Human-readable text for an fa_status value (static storage, never NULL). */
const char *fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
