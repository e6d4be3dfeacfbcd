// Internal interface between the C-ABI layer (fa_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Smallest number of query rows any kernel gives one workgroup (bounds the grid size).
constexpr int kBlockM = 128;
// Key ranges of a split forward are multiples of this many keys, so every
// kernel's key tile divides them.
constexpr int kSplitQuantum = 64;

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    float *o_part;    // split forward: fp32 partial outputs [nsplit][B][Hq][Nq][d]
    float *lse_part;  // split forward: partial log-sum-exp   [nsplit][B][Hq][Nq]
    int B, Hq, Hkv;
    int Nq, Nk;       // query and key sequence lengths
    int off;          // Nk - Nq: key j is visible to query i (causal) iff j <= i + off
    int group;        // Hq / Hkv: query heads sharing one key/value head
    int ntiles;       // query tiles per (batch, head); set by each kernel's launcher
    int nsplit;       // key ranges per query tile (1: the whole key sequence)
    int split_keys;   // keys per range, a multiple of kSplitQuantum
    int causal;
    int xcd_groups;   // 1 when B*Hkv is a multiple of 8 (one XCD per head group)
    int qmode;        // 0: q as given; 1: q negated (scale < 0); 2: q zeroed (scale == 0)
    float c;          // |scale| * log2(e) (positive), or 1 when scale == 0
    // fp8 forward: dequantisation factors per (batch, head), real value = code * factor
    const float *q_descale;   // [B][Hq]
    const float *k_descale;   // [B][Hkv]
    const float *v_descale;   // [B][Hkv]
    // fp8 forward with per-block scales (NULL: per (batch, head) descales above):
    // real value = code * 2^exp, one exp per 64 rows of a head
    const int8_t *q_exp;      // [B][Hq][ceil(Nq / 64)]
    const int8_t *k_exp;      // [B][Hkv][ceil(Nk / 64)]
    const int8_t *v_exp;      // [B][Hkv][ceil(Nk / 64)]
    // block-sparse forward: mask [Hq][mask_nqb][mask_nkb] over 128 query rows x 64 keys (NULL: dense)
    const uint8_t *block_mask;
    int mask_nqb, mask_nkb;
};

// Debug build switch (FA_SINGLE_STAGE=1): the bf16 and fp8 forward kernels
// keep one K/V LDS stage and the backward kernels one K/V (dQ) and one Q/dO
// (dK/dV) stage.  A tile is loaded only after the barrier that ends every
// read of the stage, and read only after its loads have completed and a
// barrier: no load overlaps a read.  The arithmetic and its order are those
// of the normal (double-buffered) build, so the outputs must be equal bit
// for bit; a difference points at a missing wait or barrier.
#ifndef FA_SINGLE_STAGE
#define FA_SINGLE_STAGE 0
#endif
constexpr bool kSingleStage = FA_SINGLE_STAGE != 0;
// the stage count each kernel source was built with (1 or 2)
int fwd_bf16_lds_stages();
int fwd_fp8_lds_stages();
int fwd_f32_lds_stages();
int bwd_lds_stages();

hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams &p, int d, hipStream_t stream);
// Few query rows per K/V head (decoding): rows of one head group packed into
// 32-row blocks, K/V read once per group.
hipError_t launch_decode_bf16(const FwdParams &p, int d, hipStream_t stream);
constexpr int kDecodeRowBlock = 32;
// Packed rows (query rows x query heads per K/V head) up to which the
// decoding kernel is used for bf16.
constexpr int kDecodeMaxRows = 64;
inline bool use_decode(int Nq, int group) { return (int64_t)Nq * group <= kDecodeMaxRows; }
hipError_t launch_fwd_f32(const FwdParams &p, int d, hipStream_t stream);
struct BwdParams {
    const void *q, *k, *v, *o, *dout;   // bf16 inputs (o: the forward's output)
    const float *lse;                   // the forward's log-sum-exp [B][Hq][Nq]
    float *delta;                       // workspace: rowsum(dO * O) [B][Hq][Nq]
    float *lse2;                        // workspace: lse * log2(e), +inf for rows without keys [B][Hq][Nq]
    void *dq, *dk, *dv;                 // bf16 outputs
    int B, Hq, Hkv, Nq, Nk;
    int off;                            // Nk - Nq (bottom-right causal alignment)
    int group;                          // Hq / Hkv
    int causal;
    int xcd_groups;                     // 1 when B*Hkv is a multiple of 8
    int qmode;                          // as in FwdParams (q or k negated / zeroed for the scale's sign)
    float c;                            // |scale| * log2(e), or 1 when scale == 0
    float scale;                        // the signed scale (dq = scale dS K, dk = scale dS^T Q)
};
hipError_t launch_bwd_bf16(const BwdParams &p, int d, hipStream_t stream);

// Block-scaled e4m3 quantisation (fa_quant_fp8.hip): rows per block, and
// the arguments.
constexpr int kQuantBlock = 64;
struct QuantParams {
    const void *x;          // bf16 [B][N][H][128]
    void *codes;            // e4m3 [B][N][H][128]
    int8_t *exps;           // [B][H][ceil(N / 64)]: block value = code * 2^exp
    const int8_t *signs;    // [128] of +-1 (rotation), or NULL (none)
    int B, N, H;
};
hipError_t launch_quant_fp8(const QuantParams &p, hipStream_t stream);

// The bf16 split forward in two parts (fa_api.cpp), for entry points that
// bring their own scratch memory: validation of every argument and the
// workspace size it needs (0 without a split), then the launches with the
// workspace at ws.
int splitkv_prepare(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                    int Nq, int Nk, int d, float scale, int causal, int num_splits, FwdParams &p,
                    size_t &ws_need);
int splitkv_run(FwdParams &p, int d, void *ws, hipStream_t stream);

// Merge of the nsplit partial results into o (bf16 when out_bf16, else fp32) and lse.
hipError_t launch_combine(const FwdParams &p, int d, int out_bf16, hipStream_t stream);

// Workgroup index -> (batch, query head, query tile, key range).
//
// Workgroups are dealt to the 8 XCDs round-robin by index, so index L runs
// on XCD L % 8.  When B*Hkv is a multiple of 8, XCD x is given every query
// tile of the key/value head groups g with g % 8 == x (all query heads that
// share a K/V head included), so the K/V of a head is fetched into one XCD's
// L2 only.  Within an XCD, causal tiles go heaviest first (the last query
// tile sees the most keys), which keeps the tail of the launch short.  The
// key ranges of one query tile are adjacent in the order.
__device__ __forceinline__ void decode_tile(const FwdParams &p, int &b, int &h, int &tile, int &split)
{
    const int L = blockIdx.x;
    int t;
    if (p.xcd_groups) {
        const int xcd = L & 7, s = L >> 3;
        const int heads_here = (p.B * p.Hkv >> 3) * p.group;
        const int per_t = heads_here * p.nsplit;
        t = s / per_t;
        int r = s - t * per_t;
        split = r / heads_here;
        r -= split * heads_here;
        const int lg = r / p.group, qh = r - lg * p.group;
        const int g = lg * 8 + xcd;
        b = g / p.Hkv;
        h = (g - b * p.Hkv) * p.group + qh;
    } else {
        const int per = p.B * p.Hq;
        const int per_t = per * p.nsplit;
        t = L / per_t;
        int r = L - t * per_t;
        split = r / per;
        r -= split * per;
        b = r / p.Hq;
        h = r - b * p.Hq;
    }
    tile = p.causal ? (p.ntiles - 1 - t) : t;
}

// Key tiles [lo, hi) of width BN that the workgroup with query rows
// [q_first, q_first + rows) and key range `split` visits: the range's tiles,
// cut (causal) after the tile holding the last key its last row can see.
// hi <= lo means none.
template <int BN>
__device__ __forceinline__ void key_tiles(const FwdParams &p, int q_first, int rows, int split, int &lo, int &hi)
{
    const int per = p.split_keys / BN;
    lo = split * per;
    hi = min((p.Nk + BN - 1) / BN, lo + per);
    if (p.causal) {
        const int last = min(q_first + rows, p.Nq) - 1 + p.off;   // last key any row here sees
        hi = last < 0 ? lo : min(hi, last / BN + 1);
    }
}

}  // namespace fa
