// Fused exact attention forward with fp8 (OCP e4m3) Q, K, V, bf16 output,
// fp32 accumulation and statistics, on the CDNA4 (gfx950) fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4).  Two scale granularities: one fp32
// factor per (batch, head), folded into the score scale and the output, or
// one power of two per 64 rows of Q, K and V, which the products apply
// through their block-scale operands (fa_fwd_fp8_block).
//
// The low-precision forward of the second page ("FlashAttention：IO 感知的精确
// 注意力", section 10 on FlashAttention-3's FP8 path and section 12.2 on
// per-block scales): Q, K and V arrive as e4m3 codes with one dequantisation
// factor per (batch, head), which the kernel folds into the score scale and
// the output; the probabilities are re-quantised to e4m3 for the P V
// product.  Everything else is the bf16 kernel's algorithm and schedule
// (fa_fwd_bf16.hip): Q-block-outer FlashAttention-2 loop, online softmax with
// the single division at the end, causal tiles above the diagonal skipped,
// eight wavefronts in two groups one phase apart ("ping-pong" of matrix and
// softmax phases), K/V tiles double-buffered in LDS by direct buffer loads.
//
// Differences forced by the 8-bit format:
//  * One 32x32x64 product covers 64 elements of the contraction.  Lane half
//    hf of both operands holds contraction slots 32*hf + 0..31 (measured:
//    byte j of lane half hf of A meets byte j of the same half of B).  Q and
//    K rows therefore enter as 32 consecutive bytes; for P V the 64 keys of a
//    tile are ordered so that byte j of lane half hf is key
//    16*(j/8) + 8*hf + (j%8), which is where the two 32-key score blocks
//    left them, and V^T is read with ds_read_b64_tr_b8 (within 16 lanes,
//    lane i receives byte i of each of the 8 consecutive 16-byte rows the
//    group addresses).
//  * e4m3 holds at most 448, so the probabilities are taken against an exact
//    running maximum (updated when a tile's maximum exceeds it by more than
//    one base-2 unit) and scaled by 2^7: P' = 2^(s*c - m + 7) <= 256, and
//    values down to 2^-17 of the maximum keep a code.
//  * The sum of the quantised probabilities, which normalises O (so that O
//    stays a convex combination of the V rows), comes from the matrix cores:
//    one 16x16x128 product per tile whose B operand is the P'^T register set
//    of the P V products and whose A operand is a 0/1 selector (below).  The
//    sum of e4m3 values is exact in fp32 in any order.  The fp32 sum of the
//    unquantised values gives the log-sum-exp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

constexpr int D = 128;          // head dimension (the only one this kernel takes)
constexpr int kBM = 256;        // query rows per workgroup: 8 wavefronts x 32
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 512;
constexpr float kBias = 7.0f;   // P' = 2^(s*c - m + kBias)
constexpr float kLazy = 1.0f;   // running maximum moves when a tile exceeds it by more than this
constexpr float kLn2 = 0.693147180559945309f;
// A compile-time integer passed as an argument to a generic lambda.
template <int V> struct ic { static constexpr int value = V; };

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same product with block scales 2^(sa - 127) on A and 2^(sb - 127) on B
// (E8M0 codes in the low byte).  Measured lane layout: the scale of operand
// row (A) or column (B) i over contraction half h comes from lane i + 32 h,
// the lane that holds that half of the row or column.
__device__ __forceinline__ f32x16_t mfma_fp8_scaled(i32x8_t a, i32x8_t b, f32x16_t c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ f32x4_t mfma16_fp8(i32x8_t a, i32x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Four floats -> four e4m3 codes (round to nearest even) in one dword: c, d
// into the high half, then a, b into the low half.  The first conversion
// keeps the other half of the dword it is given; giving it c's own bits
// (c is dead after it) spares a register cleared for the purpose.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_bit_cast(int, c), true);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
}

__device__ __forceinline__ float max_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte chunk permutations (a row is 8 chunks).  K: the 16 rows one phase
// of a 16-byte operand read touches land in distinct bank groups.  V: the 8
// rows x 2 chunks one phase of the 8-bit transpose read touches do.
__device__ __forceinline__ int k_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int v_swz(int row) { return 2 * ((row >> 1) & 3); }

__device__ __forceinline__ void load_lds16(const void *base, int range, uint32_t off, lds_void_t *dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void lds_wait_vm()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier that leaves this wavefront's global-to-LDS loads in
// flight (__syncthreads() would wait for them): only its LDS accesses
// complete first.  One asm statement with a memory clobber, so no LDS access
// moves across it.
__device__ __forceinline__ void barrier_keep_loads()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// BLK: per-block scales (one power of two per 64 rows of Q, K and V, applied
// by the products themselves) instead of one factor per (batch, head).
template <bool CAUSAL, bool BLK>
__global__ void __launch_bounds__(kThreads, 1) fwd_fp8_kernel(FwdParams p)
{
    constexpr int KSTEPS = D / 64;                 // K-steps of S^T = K Q^T
    constexpr int XB = D / 32;                     // 32-row blocks of O^T
    constexpr int NKB = kBN / 32;                  // 32-key blocks per tile
    constexpr int ROW_BYTES = D;
    constexpr int CHUNKS = D / 16;
    constexpr int ROWS_PER_BLK = 1024 / ROW_BYTES; // rows per 1 KB direct-load block
    constexpr int TILE = kBN * ROW_BYTES;          // bytes per tile
    static_assert(TILE / 1024 == kThreads / 64, "one direct-load block per wavefront and tile");

    __shared__ __attribute__((aligned(1024))) uint8_t Ks0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Ks1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs1[TILE];

    int b, h, tile, split;
    decode_tile(p, b, h, tile, split);
    const int hk = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2;
    const int lq = lane & 31, hf = lane >> 5;
    const int N = p.Nq;
    const int q_first = tile * kBM;
    const int wq0 = __builtin_amdgcn_readfirstlane(q_first + wave * 32);
    const int my_q = wq0 + lq;
    // score scale in base 2 with both dequantisation factors folded in (per
    // (batch, head)); with block scales the products apply them instead
    const float c = BLK ? p.c : p.c * p.q_descale[b * p.Hq + h] * p.k_descale[b * p.Hkv + hk];
    const float vscale = BLK ? 1.f : p.v_descale[b * p.Hkv + hk];
    // block scales as E8M0 codes: Q's for this wavefront's 32 rows (they lie
    // in one 64-row block), K's and V's per 64-key tile (kQuantBlock == kBN)
    static_assert(kQuantBlock == kBN && kQuantBlock % 32 == 0, "one scale per key tile");
    const int nbq = (N + kQuantBlock - 1) / kQuantBlock;
    const int8_t *kexp = BLK ? p.k_exp + (int64_t)(b * p.Hkv + hk) * nbq : nullptr;
    const int8_t *vexp = BLK ? p.v_exp + (int64_t)(b * p.Hkv + hk) * nbq : nullptr;
    const int sq = BLK ? 127 + p.q_exp[(int64_t)(b * p.Hq + h) * nbq + min(wq0 / kQuantBlock, nbq - 1)] : 127;

    const int sQ = p.Hq * D, sK = p.Hkv * D;
    const uint8_t *qbase = (const uint8_t *)p.q + ((int64_t)b * N * p.Hq + h) * D;
    const uint8_t *kbase = (const uint8_t *)p.k + ((int64_t)b * N * p.Hkv + hk) * D;
    const uint8_t *vbase = (const uint8_t *)p.v + ((int64_t)b * N * p.Hkv + hk) * D;
    const int range = N * sK;

    // ---- Q^T operand: lane (lq, hf) holds q[my_q][64t + 32hf .. +31] for step t
    i32x8_t qreg[KSTEPS];
    if (my_q < N && p.qmode != 2) {
        const i32x8_t *src = (const i32x8_t *)(qbase + (int64_t)my_q * sQ);
        const int flip = p.qmode == 1 ? (int)0x80808080u : 0;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            qreg[t] = src[2 * t + hf];
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[t][e] ^= flip;
        }
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[t][e] = 0;
    }

    int n = (N + kBN - 1) / kBN;
    if (CAUSAL) n = (min(q_first + kBM, N) - 1) / kBN + 1;
    const bool wave_live = wq0 < N;
    auto visible = [&](int j) __attribute__((always_inline)) { return wave_live && (!CAUSAL || j * kBN <= wq0 + 31); };

    // ---- HBM -> LDS: one 1 KB block per wavefront and tile; lane l fills
    // physical chunk l % CHUNKS of row l / CHUNKS of the block
    const int ld_row = wave * ROWS_PER_BLK + lane / CHUNKS, ld_pch = lane % CHUNKS;
    auto load_k = [&](int j, uint8_t *dst) {
        const uint32_t off = (uint32_t)(j * kBN + ld_row) * (uint32_t)sK + ((ld_pch ^ k_swz(ld_row)) * 16);
        load_lds16(kbase, range, off, (lds_void_t *)&dst[wave * 1024]);
    };
    auto load_v = [&](int j, uint8_t *dst) {   // the single-stage build's V loads
        const uint32_t off = (uint32_t)(j * kBN + ld_row) * (uint32_t)sK + ((ld_pch ^ v_swz(ld_row)) * 16);
        load_lds16(vbase, range, off, (lds_void_t *)&dst[wave * 1024]);
    };
    // Tile loads of an even phase: the leading group's four wavefronts move
    // two 1 KB blocks of K_{j+1} and two of V_j each at the start of their
    // matrix-core step (with all eight wavefronts loading one block each at
    // the start of the phase, the phase ran 7% slower), as straight-line code
    // (a tile that does not exist goes through a zero-length range).
    const int wl4 = __builtin_amdgcn_readfirstlane(wave & 3);
    uint32_t k_off2[2], v_off2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (wl4 * 2 + i) * ROWS_PER_BLK + lane / CHUNKS;
        k_off2[i] = (uint32_t)row * (uint32_t)sK + ((ld_pch ^ k_swz(row)) * 16);
        v_off2[i] = (uint32_t)row * (uint32_t)sK + ((ld_pch ^ v_swz(row)) * 16);
    }
    auto issue_kv = [&](int jl, uint8_t *knext, uint8_t *vnext) __attribute__((always_inline)) {
        const int krange = jl + 1 < n ? range : 0, vrange = jl < n ? range : 0;
        const uint32_t ks = (uint32_t)((jl + 1) * kBN) * (uint32_t)sK, vs = (uint32_t)(jl * kBN) * (uint32_t)sK;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            load_lds16(kbase, krange, k_off2[i] + ks, (lds_void_t *)&knext[(wl4 * 2 + i) * 1024]);
            load_lds16(vbase, vrange, v_off2[i] + vs, (lds_void_t *)&vnext[(wl4 * 2 + i) * 1024]);
        }
    };

    const int krow = (lq & 0x13) | ((lq & 4) << 1) | ((lq & 8) >> 1);
    // 8-bit transpose reads: lane group tg, lane ts within it
    const int tg = lane >> 4, ts = lane & 15;
    const int tr_row = 8 * (tg >> 1) + (ts >> 1);   // + 16 jb
    const int tr_chunk = tg & 1;                    // + 2 xb
    const int tr_byte = 8 * (ts & 1);
    // Row-sum selector.  Read as the B operand of a 16x16x128 product, lane
    // l's P'^T bytes are 32 keys of query l % 32, i.e. query n + 16 (g % 2)
    // for column n = l % 16 and K group g = l / 16.  The A operand holds e4m3
    // 1.0 where the K group's parity equals that of the output row block
    // (rows 4r .. 4r+3, r = row / 4) and 0 elsewhere, so every accumulator
    // register of lane l receives the sum over all 64 keys of its own query
    // l % 32.
    const int sel_w = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;
    const i32x8_t sum_sel = {sel_w, sel_w, sel_w, sel_w, sel_w, sel_w, sel_w, sel_w};

    float m_run = -INFINITY;   // running maximum (base 2), shared by both halves
    float l_run = 0.f;         // fp32 sum of this half's unquantised probabilities
    f32x16_t oacc[XB];         // O^T
    f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};   // the sum of the quantised probabilities
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[xb][i] = 0.f;
    f32x16_t sacc[NKB];
    i32x8_t pb;                // P'^T (e4m3) of the tile whose product is next

    // Matrix-core step for tile j: S_j^T = K_j Q^T first (the next softmax
    // step reads it at once), then O^T += V_{j-1}^T P_{j-1}^T and the sum of
    // the quantised probabilities.
    auto mfma_step = [&](int j, const uint8_t *kcur, const uint8_t *vprev, int sk, int sv) __attribute__((always_inline)) {
        if (j < n && visible(j)) {
            const char *ks = (const char *)kcur;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
                const int row = kb * 32 + krow;
                const char *kr = ks + row * ROW_BYTES;
                const int sw = k_swz(row);
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    const u32x4_t lo = *(const u32x4_t *)(kr + (((4 * t + 2 * hf) ^ sw) * 16));
                    const u32x4_t hi = *(const u32x4_t *)(kr + (((4 * t + 2 * hf + 1) ^ sw) * 16));
                    const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    sacc[kb] = BLK ? mfma_fp8_scaled(a, qreg[t], sacc[kb], sk, sq) : mfma_fp8(a, qreg[t], sacc[kb]);
                }
            }
        }
        if (j >= 1 && visible(j - 1)) {
            const char *vs = (const char *)vprev;
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                i32x8_t a;
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    const int row = 16 * jb + tr_row;
                    const int off = row * ROW_BYTES + (((2 * xb + tr_chunk) ^ v_swz(row)) * 16) + tr_byte;
                    const i32x2_t t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t *)(vs + off));
                    a[2 * jb] = t2[0];
                    a[2 * jb + 1] = t2[1];
                }
                oacc[xb] = BLK ? mfma_fp8_scaled(a, pb, oacc[xb], sv, 127) : mfma_fp8(a, pb, oacc[xb]);
            }
            lacc = mfma16_fp8(sum_sel, pb, lacc);
        }
    };

    auto softmax_step = [&](int j) __attribute__((always_inline)) {
        if (!visible(j)) return;
        const int key0 = j * kBN;
        if ((key0 + kBN > N) || (CAUSAL && key0 + kBN - 1 > wq0)) {
            const int lim = (CAUSAL ? min(my_q, N - 1) : N - 1) - (key0 + 8 * hf);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb * 32 + 16 * (i >> 3) + (i & 7) > lim) sacc[kb][i] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        const float m_tile = max_halves(mx) * c;
        const bool grow = m_tile > m_run + kLazy;
        float alpha = 1.f;
        if (grow) {
            alpha = __builtin_amdgcn_exp2f(m_run - m_tile);   // 0 on the first visit
            m_run = m_tile;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) oacc[xb] *= alpha;
            lacc[0] *= alpha;
        }
        const float m_sub = (m_run == -INFINITY ? 0.f : m_run) - kBias;
        float rf0 = 0.f, rf1 = 0.f;
        // byte j of lane half hf = key 16*(j/8) + 8*hf + (j%8) = register j%16 of block j/16
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kb = w >> 2, i0 = (w & 3) * 4;
            float e[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) e[z] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i0 + z], c, -m_sub));
            rf0 = w == 0 ? e[0] + e[2] : rf0 + (e[0] + e[2]);   // from the first pair, not from +0
            rf1 = w == 0 ? e[1] + e[3] : rf1 + (e[1] + e[3]);
            pb[w] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
        l_run = l_run * alpha + (rf0 + rf1);
    };

    // ---- ping-pong schedule (see fa_fwd_bf16.hip)
    if (n > 0) load_k(0, Ks0);
    lds_wait_vm();
    __syncthreads();
    const int nphase = 2 * n + 2;
    // Block-scale codes of the tiles, kept per stage like the tiles: sk0/sk1
    // for K_j (j even/odd), sv0/sv1 for V_j.  Each is read by a scalar load of
    // the aligned dword that holds it (that dword lies within the array's own
    // page): a vector load would share its wait counter with the tile loads
    // issued beside it, so that waiting for the code would wait for the tiles.
    typedef __attribute__((address_space(4))) const int const_int_t;
    auto code_at = [&](const int8_t *e, int j) __attribute__((always_inline)) -> int {
        const uintptr_t a = (uintptr_t)(e + j);
        const int w = *(const_int_t *)(a & ~(uintptr_t)3);
        return 127 + (int)(int8_t)(w >> (8 * (int)(a & 3)));
    };
    int sk0 = 127, sk1 = 127, sv0 = 127, sv1 = 127;
    if (BLK && n > 0) sk0 = code_at(kexp, 0);
    // G: the wavefront's group; P: the parity of global phase t (both
    // compile-time, so that each group's loop is straight-line code).
    auto phase = [&](auto G, auto P, int t, const uint8_t *kcur, const uint8_t *vprev, uint8_t *knext,
                     uint8_t *vnext, const int &skc, const int &svp, int &skn, int &svn) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value, par = decltype(P)::value;
        if constexpr (par == 0 && g == 0 && !kSingleStage) issue_kv(t >> 1, knext, vnext);
        if constexpr (par == 0 && !kSingleStage) {
            if (BLK) {
                const int j = t >> 1;
                if (j + 1 < n) skn = code_at(kexp, j + 1);
                if (j < n) svn = code_at(vexp, j);
            }
        }
        constexpr bool MSTEP = ((par - g) & 1) == 0;
        const int s = t - g;
        if (s >= 0 && s <= 2 * n) {
            if constexpr (MSTEP) {
                __builtin_amdgcn_s_setprio(1);
                mfma_step(s >> 1, kcur, vprev, skc, svp);
                __builtin_amdgcn_s_setprio(0);
            } else {
                softmax_step(s >> 1);
            }
        }
        if constexpr (par == 1) {            // the next tiles resident before the next even phase
            lds_wait_vm();
            __syncthreads();
        } else {                             // they may still be arriving
            barrier_keep_loads();
        }
    };
    auto run = [&](auto G) __attribute__((always_inline)) {
        if constexpr (kSingleStage) {
            for (int t = 0; t < nphase; t += 2) {
                // The barrier after phase t - 1 ended every read of the stage
                // (K_0 and its code were loaded before the loop).
                const int j = t >> 1;
                if (j >= 1) {
                    if (j < n) load_k(j, Ks0);
                    load_v(j - 1, Vs0);
                    if (BLK) {
                        if (j < n) sk0 = code_at(kexp, j);
                        sv0 = code_at(vexp, j - 1);
                    }
                    lds_wait_vm();
                    __syncthreads();
                }
                phase(G, ic<0>(), t, Ks0, Vs0, Ks1, Vs1, sk0, sv0, sk1, sv1);
                phase(G, ic<1>(), t + 1, Ks0, Vs0, Ks1, Vs1, sk0, sv0, sk1, sv1);
            }
            return;
        }
        for (int t = 0; t < nphase; t += 4) {
            phase(G, ic<0>(), t, Ks0, Vs1, Ks1, Vs0, sk0, sv1, sk1, sv0);
            phase(G, ic<1>(), t + 1, Ks0, Vs1, Ks1, Vs0, sk0, sv1, sk1, sv0);
            if (t + 2 < nphase) {
                phase(G, ic<0>(), t + 2, Ks1, Vs0, Ks0, Vs1, sk1, sv0, sk0, sv1);
                phase(G, ic<1>(), t + 3, Ks1, Vs0, Ks0, Vs1, sk1, sv0, sk0, sv1);
            }
        }
    };
    if (grp == 0) run(ic<0>());
    else run(ic<1>());

    // ---- epilogue: O = v_descale * O_acc / sum(P') (bf16), lse = (m - bias) ln2 + ln(sum P')
    const float l_tot = sum_halves(l_run);
    if (my_q < N) {
        const bool empty = l_tot == 0.f;
        const float inv = empty ? 0.f : vscale / lacc[0];
        const float lse_row = empty ? -INFINITY : (m_run - kBias) * kLn2 + logf(l_tot);
        uint16_t *orow = (uint16_t *)p.o + ((int64_t)b * N * p.Hq + h) * D + (int64_t)my_q * sQ;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int x = xb * 32 + 8 * gi + 4 * hf;
                const u32x2_t w = {pack_bf16(oacc[xb][4 * gi] * inv, oacc[xb][4 * gi + 1] * inv),
                                   pack_bf16(oacc[xb][4 * gi + 2] * inv, oacc[xb][4 * gi + 3] * inv)};
                *(u32x2_t *)(orow + x) = w;
            }
        if (hf == 0) p.lse[((int64_t)b * p.Hq + h) * N + my_q] = lse_row;
    }
}

template <bool CAUSAL, bool BLK>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    const unsigned grid = (unsigned)p.B * (unsigned)p.Hq * (unsigned)p.ntiles;
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL, BLK>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int fwd_fp8_lds_stages() { return kSingleStage ? 1 : 2; }

hipError_t launch_fwd_fp8(const FwdParams &p_in, int d, hipStream_t stream)
{
    if (d != D) return hipErrorInvalidValue;
    FwdParams p = p_in;
    p.ntiles = (p.Nq + kBM - 1) / kBM;
    if (p.q_exp)
        return p.causal ? launch_one<true, true>(p, stream) : launch_one<false, true>(p, stream);
    return p.causal ? launch_one<true, false>(p, stream) : launch_one<false, false>(p, stream);
}

}  // namespace fa
