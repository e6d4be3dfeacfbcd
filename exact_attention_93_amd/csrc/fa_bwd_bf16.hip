// Attention backward, bf16 in / bf16 out, fp32 accumulation, on CDNA4
// (gfx950) matrix cores.
//
// Gradients of O = softmax(scale Q K^T [+ causal mask]) V for an upstream
// gradient dO, with P recomputed from the row log-sum-exp the forward
// stored, never read from memory ("[Attention优化] 从Online-Softmax到
// FlashAttention V1/V2/V3", sections 0x04 and 0x05; "FlashAttention：IO 感知的
// 精确注意力", section 6):
//     P = exp(scale Q K^T - lse),  dP = dO V^T,  delta_i = sum_x dO_ix O_ix,
//     dS = P o (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// (delta_i equals sum_j P_ij dP_ij, the softmax Jacobian term, because
// O_i = sum_j P_ij v_j.)
//
// Two kernels.  The first is Q-outer like the forward: a workgroup owns 128
// query rows of one head, computes delta for them (stored for the second
// kernel) and streams the visible K/V tiles, accumulating dQ in registers.
// The second is K/V-outer, the loop order the first page gives for the
// FlashAttention-2 backward: a workgroup owns 128 keys of one K/V head,
// holds K and V in registers and streams the query tiles (of every query
// head of the group, so grouped-query attention needs no reduction across
// workgroups), accumulating dK and dV in registers.  The pages accumulate dQ
// across the K/V-outer workgroups with atomic additions instead; here dQ
// gets its own pass, which costs one more score product per tile but keeps
// the result deterministic and avoids a float atomic per dQ element for
// every (query tile, key tile) pair.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16): as in the forward, each
// product is arranged so that one operand comes from registers and the
// other from LDS, and the accumulator of one product feeds the next as its
// B operand: first kernel S^T = K Q^T, dP^T = V dO^T (lane = query) and
// dQ^T += K^T dS^T; second kernel S = Q K^T, dP = dO V^T (lane = key),
// dV^T += dO^T P and dK^T += Q^T dS.  The rows of the LDS operand of the
// first two products are taken in the order that swaps bits 2 and 3 of the
// row index, so that accumulator register i of lane half hf holds row
// 16*(i/8) + 8*hf + (i%8), the K-slot order of the next product's B operand.
// Transposed operands are read with ds_read_b64_tr_b16.  LDS tiles are read
// both ways, so their 16-byte chunks are permuted by one XOR that is
// conflict-free for 16-byte row reads and for the transpose reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc, false);
}

__device__ __forceinline__ float sum_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Chunk permutation of every LDS tile here: conflict-free for a 16-byte
// operand read of 16 consecutive rows and for one transpose-read phase
// (4 consecutive rows x 4 consecutive chunks).
template <int D> __device__ __forceinline__ int swz(int row)
{
    return D == 128 ? (4 * (row & 3) | ((row >> 2) & 3)) : (4 * ((row >> 1) & 1) | ((row >> 2) & 3));
}

// 16 bytes per lane from base + soff + voff (bytes) into LDS at dst + 16*lane;
// soff is the wavefront-uniform part of the offset.
__device__ __forceinline__ void load_lds16(const void *base, int range, uint32_t voff, uint32_t soff, lds_void_t *dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *base, int range, uint32_t off, lds_void_t *dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, off, 0, 0, 0);
}

__device__ __forceinline__ void vm_wait_all()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A scheduling group of n LDS reads (n in 0..3, known once loops are unrolled).
__device__ __forceinline__ void ds_group(int n)
{
    if (n >= 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    else if (n == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else if (n == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}

// A rows of the first two products: bits 2 and 3 of the lane's row swapped.
__device__ __forceinline__ int perm_row(int l) { return (l & 0x13) | ((l & 4) << 1) | ((l & 8) >> 1); }

// Transposed operand from an LDS tile [rows][D] (bf16, chunks permuted by swz):
// lane i of each 16-lane group gets rows r0 + 16u + 8*(i/16 & 2)/2 ... as laid
// out for the A operand of a 32x32x16 product: A[x][k] = tile[16u + k][32xb + x].
template <int D>
__device__ __forceinline__ u32x4_t tr_operand(const char *tile, int u, int xb, int lane)
{
    const int tg = lane >> 4, ts = lane & 15;
    const int tr_row = 8 * (tg >> 1) + (ts >> 2);
    const int tr_chunk = 2 * (tg & 1) + ((ts & 3) >> 1);
    const int tr_byte = 8 * (ts & 1);
    u32x4_t a;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 16 * u + 4 * r + tr_row;
        const int off = row * (D * 2) + (((4 * xb + tr_chunk) ^ swz<D>(row)) * 16) + tr_byte;
        const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + off));
        const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
        a[2 * r] = t2[0];
        a[2 * r + 1] = t2[1];
    }
    return a;
}

// 16 bytes of row `row`, logical chunk `ch`, of an LDS tile.
template <int D>
__device__ __forceinline__ u32x4_t row_chunk(const char *tile, int row, int ch)
{
    return *(const u32x4_t *)(tile + row * (D * 2) + ((ch ^ swz<D>(row)) * 16));
}

// ============================================================ dQ (Q-outer)
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(BwdParams p)
{
    constexpr int BM = 128, BN = 64;
    constexpr int KSTEPS = D / 16, XB = D / 32, NKB = BN / 32;
    constexpr int CHUNKS = D / 8, ROW_BYTES = D * 2, ROWS_PER_BLK = 1024 / ROW_BYTES;
    constexpr int BLKS = BN * ROW_BYTES / 1024, BLKS_PER_WAVE = BLKS / 4;
    constexpr int TILE = BN * D;

    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs1[TILE];

    // (batch, head, query tile): heaviest causal tiles first
    const int L = blockIdx.x;
    const int per = p.B * p.Hq;
    const int t_ord = L / per;
    const int bh = L - t_ord * per;
    const int b = bh / p.Hq, h = bh - (bh / p.Hq) * p.Hq;
    const int ntq = (p.Nq + BM - 1) / BM;
    const int tile = CAUSAL ? ntq - 1 - t_ord : t_ord;
    const int hk = h / p.group;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hf = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = p.off;
    const int q_first = tile * BM, wq0 = q_first + wave * 32, my_q = wq0 + lq;
    const float c = p.c;
    const int sK = p.Hkv * D;

    // ---- this lane's query row: Q^T and dO^T operands, delta, lse (base 2)
    u32x4_t qreg[KSTEPS], doreg[KSTEPS];
    float delta = 0.f, lse2 = INFINITY;        // +inf: P = 0 for rows without keys and past the end
    if (my_q < Nq) {
        const int64_t rowoff = (((int64_t)b * Nq + my_q) * p.Hq + h) * D;
        const u32x4_t *qs = (const u32x4_t *)((const uint16_t *)p.q + rowoff);
        const u32x4_t *ds = (const u32x4_t *)((const uint16_t *)p.dout + rowoff);
        const u32x4_t *os = (const u32x4_t *)((const uint16_t *)p.o + rowoff);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            qreg[t] = qs[2 * t + hf];
            doreg[t] = ds[2 * t + hf];
            const u32x4_t ov = os[2 * t + hf];
#pragma unroll
            for (int e = 0; e < 4; ++e) delta = dot_bf16x2(doreg[t][e], ov[e], delta);
        }
        const float l = p.lse[((int64_t)b * p.Hq + h) * Nq + my_q];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = doreg[t] = u32x4_t{0, 0, 0, 0};
    }
    delta = sum_halves(delta);
    if (hf == 0 && my_q < Nq) {
        p.delta[((int64_t)b * p.Hq + h) * Nq + my_q] = delta;
        p.lse2[((int64_t)b * p.Hq + h) * Nq + my_q] = lse2;   // for the dK/dV kernel
    }
    if (p.qmode != 0) {
        const uint32_t keep = p.qmode == 2 ? 0u : 0xffffffffu;
        const uint32_t flip = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[t][e] = (qreg[t][e] ^ flip) & keep;
    }

    // ---- key tiles: all of them, or (causal) up to the last one the tile's last row sees
    int n = (Nk + BN - 1) / BN;
    if (CAUSAL) {
        const int last = min(q_first + BM, Nq) - 1 + off;
        n = last < 0 ? 0 : min(n, last / BN + 1);
    }
    const bool wave_live = wq0 < Nq;
    auto visible = [&](int j) { return wave_live && (!CAUSAL || j * BN <= wq0 + 31 + off); };

    const uint16_t *kbase = (const uint16_t *)p.k + ((int64_t)b * Nk * p.Hkv + hk) * D;
    const uint16_t *vbase = (const uint16_t *)p.v + ((int64_t)b * Nk * p.Hkv + hk) * D;
    const int range = Nk * sK * 2;
    // Per-lane byte offsets within a tile are fixed; the tile's own offset
    // goes in as the scalar offset, and the LDS destinations are uniform.
    const int ld_row = lane / CHUNKS, ld_pch = lane % CHUNKS;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t ld_voff[BLKS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < BLKS_PER_WAVE; ++i) {
        const int row = (wave * BLKS_PER_WAVE + i) * ROWS_PER_BLK + ld_row;
        ld_voff[i] = (uint32_t)row * (uint32_t)(sK * 2) + ((ld_pch ^ swz<D>(row)) * 16);
    }
    auto load = [&](int j, uint16_t *kd, uint16_t *vd) {
        const uint32_t soff = (uint32_t)(j * BN) * (uint32_t)(sK * 2);
#pragma unroll
        for (int i = 0; i < BLKS_PER_WAVE; ++i) {
            const int blk = wave_u * BLKS_PER_WAVE + i;
            load_lds16(kbase, range, ld_voff[i], soff, (lds_void_t *)&kd[blk * 512]);
            load_lds16(vbase, range, ld_voff[i], soff, (lds_void_t *)&vd[blk * 512]);
        }
    };

    f32x16_t dqacc[XB];
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[xb][i] = 0.f;
    const int prow = perm_row(lq);
    // LDS read addresses.  The chunk permutation depends on a row only
    // through bits that every row a lane reads shares, so the row reads of
    // K and V (rows kb*32 + prow) derive from KSTEPS per-lane offsets and the
    // transposed reads of K (rows 16u + 4r + tr_row) from 2*XB, plus
    // constant row offsets.
    int rc_off[KSTEPS], tr_off[2][XB];
    {
        const int tg = lane >> 4, ts = lane & 15;
        const int tr_row = 8 * (tg >> 1) + (ts >> 2);
        const int tr_chunk = 2 * (tg & 1) + ((ts & 3) >> 1);
        const int tr_byte = 8 * (ts & 1);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) rc_off[t] = prow * (D * 2) + (((2 * t + hf) ^ swz<D>(prow)) * 16);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                const int rw = 4 * r + tr_row;
                tr_off[r][xb] = rw * (D * 2) + (((4 * xb + tr_chunk) ^ swz<D>(rw)) * 16) + tr_byte;
            }
    }
    // transposed operand A[x][k] = tile[16u + k][32xb + x] (as tr_operand)
    auto tr_read = [&](const char *tile, int u, int xb) __attribute__((always_inline)) -> u32x4_t {
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + tr_off[r][xb] + 16 * u * (D * 2)));
            const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
            a[2 * r] = t2[0];
            a[2 * r + 1] = t2[1];
        }
        return a;
    };

    // One 32-key half of the tile at a time: S^T and dP^T for those keys,
    // dS^T in bf16, then its share of dQ^T += K^T dS^T.  With MASK (tiles
    // that cross the diagonal or the end of the keys), keys past the row's
    // last visible one get P = 0; the other tiles skip the test.
    auto compute = [&](auto MASK, int j, const uint16_t *ks_, const uint16_t *vs_) __attribute__((always_inline)) {
        constexpr bool need_mask = decltype(MASK)::value;
        const char *ks = (const char *)ks_, *vs = (const char *)vs_;
        const int key0 = j * BN;
        const int lim = (CAUSAL ? min(my_q + off, Nk - 1) : Nk - 1) - (key0 + 8 * hf);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16_t s, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t) {
                const int o = rc_off[t] + kb * 32 * (D * 2);
                s = mfma_bf16(*(const u32x4_t *)(ks + o), qreg[t], s);
                dp = mfma_bf16(*(const u32x4_t *)(vs + o), doreg[t], dp);
            }
            u32x4_t dsb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float e2[2];
#pragma unroll
                    for (int z = 0; z < 2; ++z) {
                        const int i = 8 * u + 2 * w + z;
                        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -lse2));
                        if constexpr (need_mask) pv = (kb * 32 + 16 * u + 2 * w + z > lim) ? 0.f : pv;
                        e2[z] = pv * (dp[i] - delta);
                    }
                    dsb[u][w] = pack_bf16(e2[0], e2[1]);
                }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int xb = 0; xb < XB; ++xb)
                    dqacc[xb] = mfma_bf16(tr_read(ks, 2 * kb + u, xb), dsb[u], dqacc[xb]);
        }
    };

    auto step = [&](int j, const uint16_t *ks_, const uint16_t *vs_) __attribute__((always_inline)) {
        if (!visible(j)) return;
        const int key0 = j * BN;
        if ((key0 + BN > Nk) || (CAUSAL && key0 + BN - 1 > wq0 + off)) compute(std::true_type{}, j, ks_, vs_);
        else compute(std::false_type{}, j, ks_, vs_);
    };
    if (n > 0) load(0, Ks0, Vs0);
    if constexpr (kSingleStage) {
        for (int j = 0; j < n; ++j) {
            if (j > 0) {
                __syncthreads();          // every wavefront is done with tile j-1
                load(j, Ks0, Vs0);
            }
            vm_wait_all();
            __syncthreads();              // tile j resident
            step(j, Ks0, Vs0);
        }
    } else
    for (int j = 0; j < n; j += 2) {
        vm_wait_all();
        __syncthreads();                  // tile j resident; every wavefront is done with tile j-1
        if (j + 1 < n) load(j + 1, Ks1, Vs1);
        step(j, Ks0, Vs0);
        if (j + 1 < n) {
            vm_wait_all();
            __syncthreads();
            if (j + 2 < n) load(j + 2, Ks0, Vs0);
            step(j + 1, Ks1, Vs1);
        }
    }

    if (my_q < Nq) {
        uint16_t *dst = (uint16_t *)p.dq + (((int64_t)b * Nq + my_q) * p.Hq + h) * D;
        const float sc = p.scale;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int x = xb * 32 + 8 * gi + 4 * hf;
                const u32x2_t w = {pack_bf16(dqacc[xb][4 * gi] * sc, dqacc[xb][4 * gi + 1] * sc),
                                   pack_bf16(dqacc[xb][4 * gi + 2] * sc, dqacc[xb][4 * gi + 3] * sc)};
                *(u32x2_t *)(dst + x) = w;
            }
    }
}

// ====================================================== dK, dV (K/V-outer)
// One wavefront per SIMD, so the overlap of matrix products, vector-ALU
// softmax work and LDS operand reads has to come from within the wavefront.
// Each query tile (two 32-row blocks) runs as four stages, each a run of
// products with other work placed between them:
//   A: S0, dP0            | row operands of block 1, lse/delta of block 0
//   B: S1, dP1            | softmax of block 0, its transposed operands, lse/delta of block 1
//   C: dV += dO0^T P0 ... | softmax of block 1, transposed operands of block 1
//   D: dV, dK of block 1  | row operands of block 0 of the next tile
// The tile's synchronisation (its data resident, the previous buffer free)
// sits between C and D, so D's reads already come from the next tile.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 1) bwd_dkdv_kernel(BwdParams p)
{
    constexpr int BN = 128, BQ = 64;     // keys per workgroup, query rows per tile
    constexpr int KSTEPS = D / 16, XB = D / 32;
    constexpr int CHUNKS = D / 8, ROW_BYTES = D * 2, ROWS_PER_BLK = 1024 / ROW_BYTES;
    constexpr int BLKS = BQ * ROW_BYTES / 1024, BLKS_PER_WAVE = BLKS / 4;
    constexpr int TILE_BYTES = BQ * ROW_BYTES;
    // Two stages of the Q tile, the dO tile and the tile's lse2 and delta,
    // as separate arrays: a stage is always named at compile time, so the
    // compiler sees that the loads into one stage do not touch the other
    // and need not wait for them before reading it.
    __shared__ __attribute__((aligned(1024))) char Qs0[TILE_BYTES], Qs1[TILE_BYTES], Os0[TILE_BYTES], Os1[TILE_BYTES];
    // lse2 and delta: one copy per wavefront, so that every wavefront loads
    // its own with no branch around the load
    __shared__ __attribute__((aligned(16))) char Ls0[4 * BQ * 4], Ls1[4 * BQ * 4], Ds0[4 * BQ * 4], Ds1[4 * BQ * 4];
    auto stage = [&](auto S) __attribute__((always_inline)) {
        if constexpr (decltype(S)::value == 0 || kSingleStage) return std::make_tuple(Qs0, Os0, Ls0, Ds0);
        else return std::make_tuple(Qs1, Os1, Ls1, Ds1);
    };

    // (batch, K/V head, key tile); with B*Hkv a multiple of 8, every key tile
    // of a head runs on one XCD, whose L2 then serves that head's Q and dO
    const int L = blockIdx.x;
    int b, hk, kt;
    if (p.xcd_groups) {
        const int xcd = L & 7, s = L >> 3;
        const int heads_here = (p.B * p.Hkv) >> 3;
        kt = s / heads_here;
        const int g = (s - kt * heads_here) * 8 + xcd;
        b = g / p.Hkv;
        hk = g - b * p.Hkv;
    } else {
        const int per = p.B * p.Hkv;
        kt = L / per;
        const int r = L - kt * per;
        b = r / p.Hkv;
        hk = r - b * p.Hkv;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lk = lane & 31, hf = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = p.off, G = p.group;
    const int k_first = kt * BN, wk0 = k_first + wave_u * 32, my_k = wk0 + lk;
    const float c = p.c;
    const int sQ = p.Hq * D;

    // ---- this lane's key: K and V rows as B operands (K sign/zero as the scale needs)
    u32x4_t kreg[KSTEPS], vreg[KSTEPS];
    if (my_k < Nk) {
        const int64_t rowoff = (((int64_t)b * Nk + my_k) * p.Hkv + hk) * D;
        const u32x4_t *ks = (const u32x4_t *)((const uint16_t *)p.k + rowoff);
        const u32x4_t *vs = (const u32x4_t *)((const uint16_t *)p.v + rowoff);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            kreg[t] = ks[2 * t + hf];
            vreg[t] = vs[2 * t + hf];
        }
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) kreg[t] = vreg[t] = u32x4_t{0, 0, 0, 0};
    }
    if (p.qmode != 0) {
        const uint32_t keep = p.qmode == 2 ? 0u : 0xffffffffu;
        const uint32_t flip = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) kreg[t][e] = (kreg[t][e] ^ flip) & keep;
    }

    // ---- query tiles: causal rows i see key j iff i >= j - off
    const int q_lo = CAUSAL ? max(0, k_first - off) : 0;
    const int qt_lo = q_lo / BQ;
    const int qt_end = (Nq + BQ - 1) / BQ;
    const int nqt = q_lo < Nq ? qt_end - qt_lo : 0;
    const int total = G * nqt;            // (query head in group, query tile) pairs, in that order
    // Per head, the tiles in [m1, m2) need no mask for this wavefront: (causal)
    // their first row already sees all 32 of its keys, and they end inside Nq.
    const int m2 = max(qt_lo, (Nq % BQ) != 0 ? qt_end - 1 : qt_end);
    int m1 = qt_lo;
    if (CAUSAL) {
        const int need = wk0 + 31 - off;  // first row that sees every key of the wavefront
        m1 = need <= 0 ? 0 : (need + BQ - 1) / BQ;
        m1 = min(max(m1, qt_lo), m2);
    }

    const int range = Nq * sQ * 2;
    // Per-lane byte offsets within a tile are fixed; the tile's own offset
    // goes in as the scalar offset, and the LDS destinations are uniform.
    const int ld_row = lane / CHUNKS, ld_pch = lane % CHUNKS;
    uint32_t ld_voff[BLKS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < BLKS_PER_WAVE; ++i) {
        const int row = (wave * BLKS_PER_WAVE + i) * ROWS_PER_BLK + ld_row;
        ld_voff[i] = (uint32_t)row * (uint32_t)(sQ * 2) + ((ld_pch ^ swz<D>(row)) * 16);
    }
    // tile `it` (head hk*G + it/nqt, query tile qt_lo + it%nqt) into stage S = it&1
    // Issued whether or not the tile exists (it >= total loads nothing: zero
    // ranges), so that no branch separates loads from the reads after them.
    auto load = [&](auto S, int it_) __attribute__((always_inline)) {
        auto [qd, od, ld, dd] = stage(S);
        const bool live = it_ < total;
        const int it = live ? it_ : 0;
        const int hh = it / nqt, qt = qt_lo + (it - hh * nqt);
        const int h = hk * G + hh;
        const uint16_t *qb = (const uint16_t *)p.q + ((int64_t)b * Nq * p.Hq + h) * D;
        const uint16_t *ob = (const uint16_t *)p.dout + ((int64_t)b * Nq * p.Hq + h) * D;
        const uint32_t soff = (uint32_t)(qt * BQ) * (uint32_t)(sQ * 2);
#pragma unroll
        for (int i = 0; i < BLKS_PER_WAVE; ++i) {
            const int blk = wave_u * BLKS_PER_WAVE + i;
            load_lds16(qb, live ? range : 0, ld_voff[i], soff, (lds_void_t *)(qd + blk * 1024));
            load_lds16(ob, live ? range : 0, ld_voff[i], soff, (lds_void_t *)(od + blk * 1024));
        }
        // the tile's 64 lse and delta values, into this wavefront's copy
        const int64_t r0 = ((int64_t)b * p.Hq + h) * Nq;
        const int rng = live ? max(0, Nq - qt * BQ) * 4 : 0;
        load_lds4(p.lse2 + r0 + qt * BQ, rng, lane * 4, (lds_void_t *)(ld + wave_u * BQ * 4));
        load_lds4(p.delta + r0 + qt * BQ, rng, lane * 4, (lds_void_t *)(dd + wave_u * BQ * 4));
    };
    // Tile `it` resident and visible, every wavefront done with tile it-1's
    // buffer; then tile it+1 goes into that buffer.  (Called once more after
    // the last tile, so that every wavefront passes the same barriers.)
    // S is the stage of tile it+1, the one tile it-1 used.
    auto sync = [&](auto S, int it) __attribute__((always_inline)) {
        vm_wait_all();
        __syncthreads();
        load(S, it + 1);
    };
    // The single-stage build's synchronisation before tile it: every
    // wavefront done with tile it-1, then tile it loaded into the one stage
    // and resident.
    auto sync_single = [&](int it) __attribute__((always_inline)) {
        __syncthreads();
        load(std::integral_constant<int, 0>{}, it);
        vm_wait_all();
        __syncthreads();
    };

    f32x16_t dk[XB], dv[XB];
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[xb][i] = dv[xb][i] = 0.f;

    // LDS read offsets (bytes within a tile).  The chunk permutation depends
    // on a row only through bits 0..3, which every row a lane reads shares,
    // so block qb adds qb*32 rows and transpose group u adds 16u rows.
    const int prow = perm_row(lk);
    int rc_off[KSTEPS], tr_off[2][XB];
    {
        const int tg = lane >> 4, ts = lane & 15;
        const int tr_row = 8 * (tg >> 1) + (ts >> 2);
        const int tr_chunk = 2 * (tg & 1) + ((ts & 3) >> 1);
        const int tr_byte = 8 * (ts & 1);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) rc_off[t] = prow * ROW_BYTES + (((2 * t + hf) ^ swz<D>(prow)) * 16);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                const int rw = 4 * r + tr_row;
                tr_off[r][xb] = rw * ROW_BYTES + (((4 * xb + tr_chunk) ^ swz<D>(rw)) * 16) + tr_byte;
            }
    }
    // transposed operand A[x][k] = tile[16u + k][32xb + x] of a 32-row block
    auto tr_read = [&](const char *blk, int u, int xb) __attribute__((always_inline)) -> u32x4_t {
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t *)(blk + tr_off[r][xb] + 16 * u * ROW_BYTES));
            const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
            a[2 * r] = t2[0];
            a[2 * r + 1] = t2[1];
        }
        return a;
    };
    auto row_read = [&](const char *blk, int t) __attribute__((always_inline)) -> u32x4_t {
        return *(const u32x4_t *)(blk + rc_off[t]);
    };
    // lse2 and delta of the 16 rows a lane holds in a 32-row block: register i
    // holds row 16*(i/8) + 8*hf + (i%8), so four 4-float reads each
    auto stat_read = [&](const char *base, int qb, f32x4_t (&v)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                v[2 * u + h] = *(const f32x4_t *)(base + 4 * (qb * 32 + 16 * u + 8 * hf + 4 * h));
    };
    // P and dS = P (dP - delta) for the register pair (u, w) of one block
    // (rows 16u + 8hf + 2w, +1), as bf16 B-operand words.  With MASK, rows
    // past Nq and (causal) keys after the row's last visible key get P = 0.
    auto softmax_pair = [&](auto MASK, int qrow0, int u, int w, const f32x16_t &s, const f32x16_t &dp,
                            const f32x4_t (&l2)[4], const f32x4_t (&dl)[4], u32x4_t (&pb)[2], u32x4_t (&dsb)[2])
                            __attribute__((always_inline)) {
        constexpr bool M = decltype(MASK)::value;
        float pv[2], dsv[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const int e = 2 * w + z, i = 8 * u + e;
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -l2[2 * u + (e >> 2)][e & 3]));
            if constexpr (M) {
                // valid rows: lo <= 16u + e <= hi (register order within the block)
                const int hi = Nq - 1 - qrow0 - 8 * hf;
                const int lo = CAUSAL ? my_k - off - qrow0 - 8 * hf : -BQ;
                const int re = 16 * u + e;
                pe = ((re >= lo) & (re <= hi)) ? pe : 0.f;
            }
            pv[z] = pe;
            dsv[z] = pe * (dp[i] - dl[2 * u + (e >> 2)][e & 3]);
        }
        pb[u][w] = pack_bf16(pv[0], pv[1]);
        dsb[u][w] = pack_bf16(dsv[0], dsv[1]);
    };

    // Row operands of block 0 of the next tile, carried from stage D.
    u32x4_t qa0[KSTEPS], oa0[KSTEPS];
    auto read_block0 = [&](auto S) __attribute__((always_inline)) {
        auto [qs, os, ls_, ds_] = stage(S);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            qa0[t] = row_read(qs, t);
            oa0[t] = row_read(os, t);
        }
    };

    // One query tile.  Stages B and C are written as KSTEPS chunks, each two
    // products with its share of the softmax and the operand reads after
    // them, the chunks kept apart by scheduling barriers: one pair of
    // softmax registers per chunk at d = 128, two at d = 64.
    constexpr int NCH = KSTEPS, PAIRS = 8 / NCH, STATS = 8 / NCH;
    static_assert(2 * XB == NCH && 4 * XB == 2 * NCH, "two transposed operands and two products per chunk");
    // S: the tile's stage (it & 1), known at compile time.
    auto tile = [&](auto MASK, auto S, int it, int qt) __attribute__((always_inline)) {
        constexpr int SN = 1 - decltype(S)::value;
        auto [qs, os, ls, ds] = stage(S);
        // ---- A: S0, dP0 | row operands of block 1, stats of block 0
        f32x16_t s0, dp0, s1, dp1;
#pragma unroll
        for (int i = 0; i < 16; ++i) s0[i] = dp0[i] = 0.f;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            s0 = mfma_bf16(qa0[t], kreg[t], s0);
            dp0 = mfma_bf16(oa0[t], vreg[t], dp0);
        }
        u32x4_t qa1[KSTEPS], oa1[KSTEPS];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            qa1[t] = row_read(qs + 32 * ROW_BYTES, t);
            oa1[t] = row_read(os + 32 * ROW_BYTES, t);
        }
        f32x4_t l20[4], dl0[4], l21[4], dl1[4];
        stat_read(ls + wave_u * BQ * 4, 0, l20);
        stat_read(ds + wave_u * BQ * 4, 0, dl0);
#pragma unroll
        for (int i = 0; i < 2 * KSTEPS; ++i) {      // 2*KSTEPS + 8 reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            ds_group(i < 8 ? 2 : 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- B: S1, dP1 | softmax of block 0, transposed operands of block 0, stats of block 1
#pragma unroll
        for (int i = 0; i < 16; ++i) s1[i] = dp1[i] = 0.f;
        u32x4_t pb0[2], dsb0[2], to0[2][XB], tq0[2][XB];
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            s1 = mfma_bf16(qa1[t], kreg[t], s1);
            dp1 = mfma_bf16(oa1[t], vreg[t], dp1);
#pragma unroll
            for (int g = PAIRS * t; g < PAIRS * (t + 1); ++g)
                softmax_pair(MASK, qt * BQ, g >> 2, g & 3, s0, dp0, l20, dl0, pb0, dsb0);
            const int u = t / XB, xb = t % XB;
            to0[u][xb] = tr_read(os, u, xb);
            tq0[u][xb] = tr_read(qs, u, xb);
#pragma unroll
            for (int r = STATS * t; r < STATS * (t + 1); ++r) {
                const int h = r & 3;
                const int o = wave_u * BQ * 4 + 4 * (32 + 16 * (h >> 1) + 8 * hf + 4 * (h & 1));
                if (r < 4) l21[h] = *(const f32x4_t *)(ls + o);
                else dl1[h] = *(const f32x4_t *)(ds + o);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- C: dV, dK of block 0 | softmax of block 1, transposed operands of block 1
        u32x4_t pb1[2], dsb1[2], to1[2][XB], tq1[2][XB];
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int u = t / XB, xb = t % XB;
            dv[xb] = mfma_bf16(to0[u][xb], pb0[u], dv[xb]);
            dk[xb] = mfma_bf16(tq0[u][xb], dsb0[u], dk[xb]);
#pragma unroll
            for (int g = PAIRS * t; g < PAIRS * (t + 1); ++g)
                softmax_pair(MASK, qt * BQ + 32, g >> 2, g & 3, s1, dp1, l21, dl1, pb1, dsb1);
            to1[u][xb] = tr_read(os + 32 * ROW_BYTES, u, xb);
            tq1[u][xb] = tr_read(qs + 32 * ROW_BYTES, u, xb);
            __builtin_amdgcn_sched_barrier(0);
        }
        // keep block 1's softmax here, ahead of the synchronisation below
        asm volatile("" : "+v"(pb1[0]), "+v"(pb1[1]), "+v"(dsb1[0]), "+v"(dsb1[1]));
        // ---- the next tile's synchronisation; then D: dV, dK of block 1 | row operands of block 0 of tile it+1
        if constexpr (kSingleStage) sync_single(it + 1);
        else sync(S, it + 1);     // tile it+2 goes into this tile's stage
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                dv[xb] = mfma_bf16(to1[u][xb], pb1[u], dv[xb]);
                dk[xb] = mfma_bf16(tq1[u][xb], dsb1[u], dk[xb]);
            }
        read_block0(std::integral_constant<int, SN>{});   // (after the last tile: values nobody uses)
#pragma unroll
        for (int i = 0; i < 2 * NCH; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // Every tile's synchronisation happens once, before it: here for the
    // first, at the end of stage C of the one before for the others.
    if (total > 0) {
        if constexpr (kSingleStage) {
            sync_single(0);
        } else {
            load(std::integral_constant<int, 0>{}, 0);
            sync(std::integral_constant<int, 1>{}, 0);
        }
        read_block0(std::integral_constant<int, 0>{});
    }
    for (int hh = 0; hh < G && nqt > 0; ++hh) {
        const int base = hh * nqt - qt_lo;
        // tiles [a, b) in pairs, so that each tile's stage is named at compile time
        auto run = [&](auto MASK, int a, int b) __attribute__((always_inline)) {
            constexpr std::integral_constant<int, 0> S0{};
            constexpr std::integral_constant<int, 1> S1{};
            int qt = a;
            if (qt < b && ((base + qt) & 1)) {
                tile(MASK, S1, base + qt, qt);
                ++qt;
            }
            for (; qt + 1 < b; qt += 2) {
                tile(MASK, S0, base + qt, qt);
                tile(MASK, S1, base + qt + 1, qt + 1);
            }
            if (qt < b) tile(MASK, S0, base + qt, qt);
        };
        run(std::true_type{}, qt_lo, m1);
        run(std::false_type{}, m1, m2);
        run(std::true_type{}, m2, qt_end);
    }

    if (my_k < Nk) {
        const int64_t rowoff = (((int64_t)b * Nk + my_k) * p.Hkv + hk) * D;
        uint16_t *dkd = (uint16_t *)p.dk + rowoff;
        uint16_t *dvd = (uint16_t *)p.dv + rowoff;
        const float sc = p.scale;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int x = xb * 32 + 8 * gi + 4 * hf;
                const u32x2_t wk = {pack_bf16(dk[xb][4 * gi] * sc, dk[xb][4 * gi + 1] * sc),
                                    pack_bf16(dk[xb][4 * gi + 2] * sc, dk[xb][4 * gi + 3] * sc)};
                const u32x2_t wv = {pack_bf16(dv[xb][4 * gi], dv[xb][4 * gi + 1]),
                                    pack_bf16(dv[xb][4 * gi + 2], dv[xb][4 * gi + 3])};
                *(u32x2_t *)(dkd + x) = wk;
                *(u32x2_t *)(dvd + x) = wv;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const BwdParams &p, hipStream_t stream)
{
    const unsigned g1 = (unsigned)p.B * (unsigned)p.Hq * (unsigned)((p.Nq + 127) / 128);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(g1), dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = (unsigned)p.B * (unsigned)p.Hkv * (unsigned)((p.Nk + 127) / 128);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(g2), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int bwd_lds_stages() { return kSingleStage ? 1 : 2; }

hipError_t launch_bwd_bf16(const BwdParams &p, int d, hipStream_t stream)
{
    if (d == 128) return p.causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return p.causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace fa
