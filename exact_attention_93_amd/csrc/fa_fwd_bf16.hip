// Fused exact attention forward, bf16 in / bf16 out, fp32 accumulation, for
// CDNA4 (gfx950) matrix cores.
//
// Algorithm: the Q-block-outer loop of FlashAttention-2 ("[Attention优化]
// 从Online-Softmax到FlashAttention V1/V2/V3", section 0x05; "Flash-attention
// 学习", section 2.2): a workgroup owns 256 query rows of one (batch, head),
// keeps them in registers, and streams every visible 64-key K/V tile through
// LDS once.  Each tile is merged with the online-softmax recurrence
// ("FlashAttention：IO 感知的精确注意力", section 5): running row maximum m,
// running sum l, and an unnormalised accumulator rescaled by exp(m_old - m_new)
// with the single division by l deferred to the end (FlashAttention-2, same
// sections).  Causal tiles that lie entirely above the diagonal are never
// visited; only tiles that cross the diagonal or the end of the sequence pay
// for the mask (first page, section 0x09).  Grouped-query attention reads the
// shared K/V head by index (same section).
//
// Work partition inside the workgroup: eight wavefronts share each K/V tile
// and each owns 32 whole query rows, so row statistics never cross
// wavefronts (the "sliced-Q" partition the pages credit to FlashAttention-2).
// The eight wavefronts form two groups of four, one wavefront of each group
// per SIMD, that run the same tile sequence one phase apart: while one
// group issues the matrix-core products of its tile, the other runs the
// softmax of its previous tile on the vector ALU, and they swap roles
// halfway through each tile.  This is the overlap of softmax with matrix products that the
// second page (section 10) describes for FlashAttention-3 ("ping-pong"),
// built from one CDNA workgroup barrier per tile instead of Hopper warp
// specialisation.
//
// Data movement: K and V tiles go from HBM straight into LDS with 16-byte
// buffer loads (buffer_load_dwordx4 ... lds), double-buffered so that the
// next tile streams in during the two phases that consume the current one.  The buffer descriptor's range
// check returns zeros for keys past the end of the sequence, so no address
// ever leaves the tensors.  Both tiles keep their natural [key][d] layout,
// with the 16-byte chunks of each row permuted by an XOR of the row index so
// that the matrix-core operand reads below hit distinct LDS banks.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, D = A*B + C, 32x32 output):
// the kernel computes the TRANSPOSED score tile S^T = K Q^T (A = K from LDS,
// B = Q^T from registers).  A 32x32 accumulator holds column (lane % 32) in
// every lane, so lane l owns query (l % 32) and 16 of the 32 keys of a block;
// the other 16 are in lane l ^ 32.  A row maximum or sum is therefore 16
// in-lane operations plus one exchange between the two lane halves
// (v_permlane32_swap).  The K rows are fed to the A operand in a permuted
// order (bits 2 and 3 of the row index swapped) so that accumulator register
// i of lane half hf holds key 16*(i/8) + 8*hf + (i%8): exactly the slots the
// B operand of the next product expects.  The probabilities then feed
// O^T = V^T P^T straight from registers (B = P^T), and the O^T accumulator
// again has one query per lane, so the rescale by exp(m_old - m_new) is a
// per-lane scalar.  The A operand V^T is read from the untransposed V tile
// with the LDS transpose read ds_read_b64_tr_b16: within each group of 16
// lanes, lane i receives element i%4 of the 8-byte rows addressed by lanes
// 4e + i/4 (e = 0..3), so pointing lane 4e+q at V[k0+e][x0+4q..x0+4q+3]
// hands lane i the four keys k0..k0+3 of column x0+i.
//
// Exponentials are taken base 2 with scale*log2(e) folded into one FMA per
// score.  The accumulator is only rescaled when some row's maximum grows by
// more than kLazyLog2 (base-2 units) over the reference value in use: the
// result does not depend on which reference value is subtracted (the softmax
// identity holds for any m, second page, section 5.1), the values stay
// bounded by 2^kLazyLog2, and the final division uses the same sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// A compile-time integer passed as an argument to a generic lambda.
template <int V> struct ic { static constexpr int value = V; };

constexpr int kBN = 64;        // keys per K/V tile
// Wavefronts per workgroup: 8 (two per SIMD, the two groups of the
// ping-pong), or 4 at d = 256, where one wavefront's Q and O^T alone take
// 192 registers and a single wavefront per SIMD gets the whole register
// file (the two groups then coincide and the phases run back to back).
template <int D> constexpr int wg_waves() { return D == 256 ? 4 : 8; }
template <int D> constexpr int wg_threads() { return 64 * wg_waves<D>(); }
template <int D> constexpr int wg_rows() { return 32 * wg_waves<D>(); }   // query rows per workgroup
constexpr float kLazyLog2 = 8.0f;
constexpr float kFarSum = 0x1p64f;   // tile row sum that signals a stale reference maximum
// Products whose V^T operands are read ahead of the matrix cores (measured:
// at d = 128 the four row-sum products that open the phase cover most of the
// LDS latency, so two suffice; d = 64 has half the products per phase and
// gains from six).  d = 256 keeps four.
template <int D> constexpr int pf_pv() { return D == 64 ? 6 : D == 128 ? 2 : 4; }
// Products whose K operands are read ahead of the matrix cores (measured: two
// at d = 64, four otherwise).
template <int D> constexpr int pf_qk() { return D == 64 ? 2 : 4; }
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// At d = 256 a wavefront owns the whole register file, and the compiler
// would then put every product in the AGPR form and copy each score tile out
// for the softmax.  These products are inline assembly with fixed register
// files instead: S^T and the K, V^T and P^T operands in VGPRs, Q^T and the
// O^T accumulator in AGPRs.  The compiler does not see their latency, so the
// gaps the hardware needs between a product and a vector instruction are
// explicit s_nop statements tied to the registers concerned (d = 256 only):
// a VALU write of P^T or Q^T read by a product needs 2 wait states (s_nop 3),
// a product's S^T read by the VALU 11 (s_nop 15), and O^T is read or
// rewritten by the VALU only after 32.  Accumulating into exactly the
// previous product's destination needs no gap.  The compiler also takes a
// product's result as written when it issues, and may copy or move those
// registers at any later point; so each run of products ends with a
// statement that waits out the gap and claims its destinations.
__device__ __forceinline__ void mma_s_first_v(f32x16_t &d, u32x4_t a, u32x4_t bq)
{
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(bq));
}
__device__ __forceinline__ void mma_s_v(f32x16_t &d, u32x4_t a, u32x4_t bq)
{
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(bq));
}
__device__ __forceinline__ void mma_o_a(f32x16_t &acc, u32x4_t a, u32x4_t b)
{
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 16x16x32 product (D = A*B + C); lane l holds row/column l % 16 of A/B and
// the K slots of group l / 16, and rows 4*(l/16) .. +3 of column l % 16 of D.
__device__ __forceinline__ f32x4_t mfma16_bf16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// acc + lo + hi of a packed bf16 pair, in fp32.
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

// v_permlane32_swap exchanges the upper lane half of its first operand with
// the lower half of its second; with x in both, the two results hold x of
// this lane and of lane ^ 32 (in some order), so a symmetric operation on
// them combines the two halves identically in every lane.
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

// Chunk permutations of the LDS tiles (chunk = 16 bytes; a row is D/8 chunks).
// K: the 16 rows one phase of a 16-byte operand read touches land in 16
// distinct bank groups.  V: the 4 rows x 4 chunks one phase of the transpose
// read touches land in 16 distinct bank groups.
// (d = 256 rows span two 256-byte bank windows; only the chunk index mod 16
// decides the bank group, so the d = 128 permutations serve.)
template <int D> __device__ __forceinline__ int k_swz(int row)
{
    return D != 64 ? (row & 15) : ((row >> 1) & 7);
}
template <int D> __device__ __forceinline__ int v_swz(int row)
{
    return D != 64 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// 16 bytes per lane from base + soff + voff (bytes) straight into LDS at
// dst + 16*lane, through a buffer descriptor whose range check returns zeros
// at or past `range` bytes.
// soff is the wavefront-uniform part of the offset.
__device__ __forceinline__ void load_lds16(const void *base, int range, uint32_t voff, uint32_t soff, lds_void_t *dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

// The same load as inline assembly, through a descriptor held in SGPRs
// (base, stride 0, `range` bytes, the same flags), to LDS byte address lds.
// The compiler does not see it write LDS and adds no waits for it: the
// caller orders it against the LDS reads with its own vmcnt waits and
// barriers.  M0 carries the LDS address and needs one wait state before
// the load.  M0 is a reserved register (a clobber entry would be ignored):
// the compiler sets it right before each instruction of its own that reads
// it, and a kernel that uses this load issues no such instruction.
__device__ __forceinline__ void load_lds16_asm(u32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds));
}

__device__ __forceinline__ void lds_wait_vm()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Block-sparse forward: query blocks of kMaskRows rows x key tiles of kBN
// keys; the workgroup visits only the tiles that one of its query blocks keeps.
constexpr int kMaskRows = 128;
constexpr int kMaxMaskTiles = 1024;   // key tiles a block-sparse call may have (N <= 65536)

template <int D, bool CAUSAL, bool SPLIT, bool SPARSE>
__global__ void __launch_bounds__(wg_threads<D>(), 1) fwd_bf16_kernel(FwdParams p)
{
    constexpr int kThreads = wg_threads<D>();
    constexpr int kBM = wg_rows<D>();
    constexpr int KSTEPS = D / 16;                 // K-steps of S^T = K Q^T
    constexpr int XB = D / 32;                     // 32-row blocks of O^T
    constexpr int NKB = kBN / 32;                  // 32-key blocks per tile
    constexpr int PVSTEPS = kBN / 16;              // K-steps of O^T = V^T P^T
    constexpr int CHUNKS = D / 8;                  // 16-byte chunks per row
    constexpr int ROW_BYTES = D * 2;
    constexpr int ROWS_PER_BLK = 1024 / ROW_BYTES; // rows per 1 KB direct-load block
    constexpr int BLKS = kBN * ROW_BYTES / 1024;   // 1 KB blocks per tile and tensor
    constexpr int NWAVES = kThreads / 64;
    constexpr int TILE_ELEMS = kBN * D;
    // Tile streams: one per workgroup, or, with a block mask and two
    // ping-pong groups, one per group.  Each group then owns one query block
    // of the mask and visits only the tiles that block keeps, with its own
    // K/V stages, loaded by its own four wavefronts.
    constexpr int NG = (SPARSE && NWAVES == 8) ? 2 : 1;
    constexpr int LOADERS = NWAVES / NG;           // wavefronts that load one stream
    constexpr int BLKS_PER_WAVE = BLKS / LOADERS;
    static_assert(BLKS_PER_WAVE >= 1 && BLKS % LOADERS == 0, "tile shape");
    static_assert(!SPARSE || wg_rows<D>() / kMaskRows == NG, "one query block of the mask per stream");

    // Two stages of K and V as four distinct objects.  Every access below
    // names its stage statically, so the compiler can see that the loads
    // filling one stage never alias the operand reads of the other and does
    // not make those reads wait for the loads in flight.
    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[NG * TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks1[NG * TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[NG * TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs1[NG * TILE_ELEMS];

    int b, h, tile, split;
    decode_tile(p, b, h, tile, split);
    const int hk = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2;                    // 0: leading group, 1: trailing group (8 wavefronts)
    const int lq = lane & 31, hf = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = p.off;
    const int q_first = tile * kBM;
    const int wq0 = __builtin_amdgcn_readfirstlane(q_first + wave * 32);   // first query row of this wavefront
    const int my_q = wq0 + lq;                    // query row owned by this lane
    const float c = p.c;

    // ---- K/V tiles this workgroup visits: n tiles from key key_lo on
    int kt_lo, kt_hi;
    key_tiles<kBN>(p, q_first, kBM, split, kt_lo, kt_hi);
    int n = max(0, kt_hi - kt_lo);
    const int key_lo = kt_lo * kBN;

    const int sQ = p.Hq * D, sK = p.Hkv * D;      // row strides (elements)
    const uint16_t *qbase = (const uint16_t *)p.q + ((int64_t)b * Nq * p.Hq + h) * D;
    const uint16_t *kbase = (const uint16_t *)p.k + ((int64_t)b * Nk * p.Hkv + hk) * D + (int64_t)key_lo * sK;
    const uint16_t *vbase = (const uint16_t *)p.v + ((int64_t)b * Nk * p.Hkv + hk) * D + (int64_t)key_lo * sK;
    // Loads cover keys key_lo..Nk-1 of this (batch, kv head): anything at or
    // past key Nk reads as zero.
    const int range = max(0, Nk - key_lo) * sK * 2;

    // ---- Q^T operand: lane (lq, hf) holds q[my_q][16t + 8hf .. +7] for step t
    u32x4_t qreg[KSTEPS];
    if (my_q < Nq) {
        const u32x4_t *src = (const u32x4_t *)(qbase + my_q * sQ);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = src[2 * t + hf];
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = u32x4_t{0, 0, 0, 0};
    }
    // The sign or zero fix for the scale, and at d = 256 the move of Q^T to
    // AGPRs, run just before the tile loop (finish_q), so that nothing waits
    // for these loads before the first tile's loads are issued.
    auto finish_q = [&]() __attribute__((always_inline)) {
        if (p.qmode != 0) {
            const uint32_t keep = p.qmode == 2 ? 0u : 0xffffffffu;
            const uint32_t flip = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) qreg[t][e] = (qreg[t][e] ^ flip) & keep;
        }
        if constexpr (D == 256) {
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t) {
                const u32x4_t v = qreg[t];
                asm("; q^T to agpr" : "=a"(qreg[t]) : "0"(v));
            }
            asm volatile("s_nop 3" : "+a"(qreg[0]));
#pragma unroll
            for (int t = 1; t < KSTEPS; ++t) asm volatile("" : "+a"(qreg[t]));
        }
    };

    // ---- block-sparse: for each stream (query block of the mask), the key
    // tiles it keeps, in order.  n becomes this wavefront's own count, and
    // n_loop the longest stream's, which sets the workgroup's phase count.
    // Built after the Q^T loads are issued, so that their latency and the
    // mask reads' overlap; the mask bytes of both streams and four 64-tile
    // chunks are read together before any of them is compacted.
    const int sg = NG == 2 ? grp : 0;             // this wavefront's stream
    __shared__ uint16_t tile_list[SPARSE ? NG : 1][SPARSE ? kMaxMaskTiles : 1];
    __shared__ int tile_count[NG];
    int n_loop = n;
    if constexpr (SPARSE) {
        if (wave == 0) {
            constexpr int CB = 4;                 // 64-tile chunks per batch
            const int qb0 = q_first / kMaskRows;
            const int nqb = p.mask_nqb;
            const uint8_t *mrow = p.block_mask + ((int64_t)h * nqb + qb0) * p.mask_nkb;
            int cnt[NG];
#pragma unroll
            for (int qb = 0; qb < NG; ++qb) cnt[qb] = 0;
            for (int base = kt_lo; base < kt_hi; base += 64 * CB) {
                bool kept[NG][CB];
                // every byte is read at a clamped, valid position first (no
                // branch between the loads), and the bounds applied after
#pragma unroll
                for (int qb = 0; qb < NG; ++qb)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int j = base + 64 * cb + lane;
                        const int qr = min(qb, nqb - 1 - qb0), jc = min(j, kt_hi - 1);
                        const uint8_t m = mrow[qr * p.mask_nkb + jc];
                        kept[qb][cb] = j < kt_hi && qb0 + qb < nqb && m != 0;
                    }
#pragma unroll
                for (int qb = 0; qb < NG; ++qb)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const uint64_t keep = __builtin_amdgcn_ballot_w64(kept[qb][cb]);
                        const int pos = cnt[qb] + (int)__builtin_amdgcn_mbcnt_hi(
                                            (uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0));
                        if (kept[qb][cb]) tile_list[qb][pos] = (uint16_t)(base + 64 * cb + lane);
                        cnt[qb] += __builtin_popcountll(keep);
                    }
            }
            if (lane == 0) {
#pragma unroll
                for (int qb = 0; qb < NG; ++qb) tile_count[qb] = cnt[qb];
            }
        }
        __syncthreads();
        n = tile_count[sg];
        if constexpr (NG == 2) n_loop = max(tile_count[0], tile_count[NG - 1]);
        else n_loop = n;
    }
    // absolute key-tile index of the j-th tile of this wavefront's stream
    auto tix = [&](int j) __attribute__((always_inline)) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tile_list[sg][j]);
        else return j;
    };

    // Tile j holds a key this wavefront can see (causal: keys <= its last
    // row + off).  A wavefront whose rows all lie past the end sees nothing.
    const bool wave_live = wq0 < Nq;
    auto visible = [&](int j) __attribute__((always_inline)) {
        return wave_live && (!CAUSAL || key_lo + tix(j) * kBN <= wq0 + 31 + off);
    };

    // ---- HBM -> LDS: each wavefront moves BLKS_PER_WAVE 1 KB blocks of a
    // tile of its stream; lane l fills physical chunk l % CHUNKS of row
    // l / CHUNKS.  The per-lane byte offsets within a tile are fixed; the
    // tile's own offset goes in as the scalar offset, and the LDS
    // destinations are wavefront-uniform.  A stream's tiles sit at element
    // offset sg * TILE_ELEMS of each stage.
    const int ld_row = lane / CHUNKS, ld_pch = lane % CHUNKS;
    const int wl = NG == 2 ? (wave & 3) : wave;   // index among the stream's loaders
    const int wl_u = __builtin_amdgcn_readfirstlane(wl);
    const int so = sg * TILE_ELEMS;               // this stream's part of a stage
    uint32_t k_voff[BLKS_PER_WAVE], v_voff[BLKS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < BLKS_PER_WAVE; ++i) {
        const int row = (wl * BLKS_PER_WAVE + i) * ROWS_PER_BLK + ld_row;
        k_voff[i] = (uint32_t)row * (uint32_t)(sK * 2) + ((ld_pch ^ k_swz<D>(row)) * 16);
        v_voff[i] = (uint32_t)row * (uint32_t)(sK * 2) + ((ld_pch ^ v_swz<D>(row)) * 16);
    }
    // With a block mask the loads are inline assembly (load_lds16_asm): the
    // two streams' pointers differ at run time, and the kernel's own waits
    // below order every load against the reads of its stage.
    const uint64_t kaddr = (uint64_t)kbase, vaddr = (uint64_t)vbase;
    const u32x4_t k_rsrc = {(uint32_t)kaddr, (uint32_t)(kaddr >> 32) & 0xffffu, (uint32_t)range, 0x00020000u};
    const u32x4_t v_rsrc = {(uint32_t)vaddr, (uint32_t)(vaddr >> 32) & 0xffffu, (uint32_t)range, 0x00020000u};
    auto load_tile = [&](const uint16_t *src, const u32x4_t &rsrc, const uint32_t *voff, int j, uint16_t *stage) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)(tix(j) * kBN) * (uint32_t)(sK * 2);
#pragma unroll
        for (int i = 0; i < BLKS_PER_WAVE; ++i) {
            uint16_t *dst = &stage[so + (wl_u * BLKS_PER_WAVE + i) * 512];
            if constexpr (SPARSE)
                load_lds16_asm(rsrc, voff[i], soff,
                               __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)dst));
            else
                load_lds16(src, range, voff[i], soff, (lds_void_t *)dst);
        }
    };
    auto load_k = [&](int j, uint16_t *stage) __attribute__((always_inline)) { load_tile(kbase, k_rsrc, k_voff, j, stage); };
    auto load_v = [&](int j, uint16_t *stage) __attribute__((always_inline)) { load_tile(vbase, v_rsrc, v_voff, j, stage); };
    // Dense streams (no block mask): the loads of even phase 2*jl, K_{jl+1}
    // and V_{jl}, are issued by the wavefronts whose matrix-core step runs in
    // that phase (the leading group; at d = 256 all four), spread among their
    // products: V blocks among the P V products, K blocks among the score
    // products.  (Issued by all eight wavefronts back to back at the start of
    // the phase, they kept each one waiting ~350 cycles per tile on the
    // vector-memory path.)  The loads are straight-line code with no branch,
    // so that they share a scheduling region with the products; a tile that
    // does not exist is "loaded" through a zero-length range, which moves no
    // data.
    constexpr bool SPREAD = !SPARSE;
    constexpr int SPREAD_LOADERS = NWAVES == 8 ? 4 : NWAVES;
    constexpr int BPL = BLKS / SPREAD_LOADERS;    // blocks per loader and tensor
    const int wl4 = __builtin_amdgcn_readfirstlane(wave & (SPREAD_LOADERS - 1));
    uint32_t k_voff4[SPREAD ? BPL : 1], v_voff4[SPREAD ? BPL : 1];
    if constexpr (SPREAD) {
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int row = (wl4 * BPL + i) * ROWS_PER_BLK + ld_row;
            k_voff4[i] = (uint32_t)row * (uint32_t)(sK * 2) + ((ld_pch ^ k_swz<D>(row)) * 16);
            v_voff4[i] = (uint32_t)row * (uint32_t)(sK * 2) + ((ld_pch ^ v_swz<D>(row)) * 16);
        }
    }
    auto issue_k = [&](int jl, uint16_t *knext) __attribute__((always_inline)) {
        const int krange = jl + 1 < n ? range : 0;
        const uint32_t soff = (uint32_t)((jl + 1) * kBN) * (uint32_t)(sK * 2);
#pragma unroll
        for (int i = 0; i < BPL; ++i)
            load_lds16(kbase, krange, k_voff4[i], soff, (lds_void_t *)&knext[(wl4 * BPL + i) * 512]);
    };
    auto issue_v = [&](int jl, uint16_t *vnext) __attribute__((always_inline)) {
        const int vrange = jl < n ? range : 0;
        const uint32_t soff = (uint32_t)(jl * kBN) * (uint32_t)(sK * 2);
#pragma unroll
        for (int i = 0; i < BPL; ++i)
            load_lds16(vbase, vrange, v_voff4[i], soff, (lds_void_t *)&vnext[(wl4 * BPL + i) * 512]);
    };

    // A-operand row for lane lq: key 32*kb + perm(lq), perm swaps bits 2 and 3.
    const int krow = (lq & 0x13) | ((lq & 4) << 1) | ((lq & 8) >> 1);
    // Transpose-read addressing for V^T: lane group g = lane / 16, s = lane % 16.
    const int tg = lane >> 4, ts = lane & 15;
    const int tr_row = 8 * (tg >> 1) + (ts >> 2);            // + 16u + 4r
    const int tr_chunk = 2 * (tg & 1) + ((ts & 3) >> 1);      // + 4xb
    const int tr_byte = 8 * (ts & 1);

    float m_run = -INFINITY;   // reference maximum (base-2 units), shared by both halves
    float l_run = 0.f;         // fp32 sum of this lane half's probabilities
    float lb_run = 0.f;        // the same sum over their bf16-rounded values
    f32x16_t oacc[XB];
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[xb][i] = 0.f;
    if constexpr (D == 256) {
#pragma unroll
        for (int xb = 0; xb < XB; ++xb) {
            const f32x16_t z = oacc[xb];
            asm("; o^T to agpr" : "=a"(oacc[xb]) : "0"(z));
        }
    }
    // d <= 128: the sum of the bf16 probabilities is taken on the matrix
    // cores, with one 16x16x32 product per 16 keys whose B operand is the same
    // P^T register quad the O^T products read.  (A v_dot2 on the vector ALU
    // waits for the matrix pipeline whenever the other wavefront of the SIMD
    // is issuing products, which is all of the softmax phase.)  Read as a
    // 16x32 B operand, lane l's quad holds keys of half (l / 32) for query
    // l % 32, i.e. query n + 16 (g % 2) for column n = l % 16 and K group
    // g = l / 16.  The 0/1 A operand selects, for output rows 4r .. 4r+3, the
    // K groups with g % 2 == r % 2, so every accumulator register of lane l
    // ends up holding the 16-key sum of its own query l % 32, both halves
    // included.  The accumulator is rescaled together with O^T.
    constexpr bool MSUM = D != 256;
    f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t sel_w = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x3f803f80u : 0u;
    const u32x4_t sum_sel = {sel_w, sel_w, sel_w, sel_w};
    f32x16_t sacc[NKB];        // S^T of the tile whose softmax is next
    u32x4_t pb[PVSTEPS];       // P^T (bf16) of the tile whose product is next
    // d = 256: 32 wait states between the last product into O^T and any
    // vector access to it.
    auto sync_acc = [&]() __attribute__((always_inline)) {
        if constexpr (D == 256) {
            asm volatile("s_nop 15\n\ts_nop 15" : "+a"(oacc[0]));
#pragma unroll
            for (int xb = 1; xb < XB; ++xb) asm volatile("" : "+a"(oacc[xb]));
        }
    };

    // d = 256: the products are inline assembly (O^T in AGPRs), which the
    // scheduling-group masks do not match, so their operand reads are placed
    // explicitly: a ring of operands read RING products ahead, and a
    // scheduling barrier after each product, so that no read slides back to
    // its product and leaves the only wavefront of the SIMD waiting on it.
    // Product order: P V by (u, xb) with xb inner; scores by (t, kb) with kb
    // inner, so that consecutive score products feed different accumulators.
    constexpr int RING = 4;
    auto vt_operand = [&](const char *vs, int i) __attribute__((always_inline)) -> u32x4_t {
        const int u = i / XB, xb = i % XB;
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 16 * u + 4 * r + tr_row;
            const int off = row * ROW_BYTES + (((4 * xb + tr_chunk) ^ v_swz<D>(row)) * 16) + tr_byte;
            const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off));
            const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
            a[2 * r] = t2[0];
            a[2 * r + 1] = t2[1];
        }
        return a;
    };
    auto k_operand = [&](const char *ks, int i) __attribute__((always_inline)) -> u32x4_t {
        const int t = i / NKB, kb = i % NKB;
        const int row = kb * 32 + krow;
        return *(const u32x4_t *)(ks + row * ROW_BYTES + (((2 * t + hf) ^ k_swz<D>(row)) * 16));
    };
    auto pv_ring = [&](const char *vs) __attribute__((always_inline)) {
        constexpr int NP = PVSTEPS * XB;
        u32x4_t ring[RING];
#pragma unroll
        for (int i = 0; i < RING; ++i) ring[i] = vt_operand(vs, i);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            mma_o_a(oacc[i % XB], ring[i % RING], pb[i / XB]);
            if (i + RING < NP) ring[i % RING] = vt_operand(vs, i + RING);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // The scores, with the phase's tile loads (LD: K_{jl+1} and V_{jl}, one
    // 1 KB block of each per two products from the start).
    auto s_ring = [&](const char *ks, auto LOADS, int jl, uint16_t *knext, uint16_t *vnext) __attribute__((always_inline)) {
        constexpr bool LD = decltype(LOADS)::value != 0;
        constexpr int NS = NKB * KSTEPS;
        const int krange = jl + 1 < n ? range : 0, vrange = jl < n ? range : 0;
        const uint32_t ksoff = (uint32_t)((jl + 1) * kBN) * (uint32_t)(sK * 2);
        const uint32_t vsoff = (uint32_t)(jl * kBN) * (uint32_t)(sK * 2);
        u32x4_t ring[RING];
#pragma unroll
        for (int i = 0; i < RING; ++i) ring[i] = k_operand(ks, i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = i / NKB, kb = i % NKB;
            if (t == 0) mma_s_first_v(sacc[kb], ring[i % RING], qreg[t]);
            else mma_s_v(sacc[kb], ring[i % RING], qreg[t]);
            if (i + RING < NS) ring[i % RING] = k_operand(ks, i + RING);
            if constexpr (LD) {
                if (i % 2 == 0 && i / 2 < BPL) {
                    const int b = i / 2;
                    load_lds16(vbase, vrange, v_voff4[b], vsoff, (lds_void_t *)&vnext[(wl4 * BPL + b) * 512]);
                    load_lds16(kbase, krange, k_voff4[b], ksoff, (lds_void_t *)&knext[(wl4 * BPL + b) * 512]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // S^T as written (the last products end within 16 wait states): from
        // here on the compiler may read, copy or move its registers.
        asm volatile("s_nop 15" : "+v"(sacc[0]), "+v"(sacc[1]));
    };

    // Matrix-core step for tile j: O^T += V_{j-1}^T P_{j-1}^T, then
    // S_j^T = K_j Q^T.  No vector-ALU work beyond operand addressing.
    // With LOADS (a compile-time ic<0 or 1>), the tile loads of the phase
    // (K_{jl+1}, V_{jl}) are spread among the products: V blocks among the
    // P V products, K blocks among the score products.
    auto mfma_step = [&](auto LOADS, int j, const uint16_t *kcur, const uint16_t *vprev, int jl,
                         uint16_t *knext, uint16_t *vnext) __attribute__((always_inline)) {
        constexpr bool LD = decltype(LOADS)::value != 0;
        if (j >= 1 && visible(j - 1)) {
            const char *vs = (const char *)(vprev + so);
            if constexpr (D == 256) {   // P^T was written by the vector ALU
                asm volatile("s_nop 3" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]));
                pv_ring(vs);
                // O^T as written, before any control-flow merge at which the
                // compiler may copy it (such a copy can follow the products
                // at once, e.g. past a barrier the other wavefronts already
                // wait at).
                sync_acc();
            } else {
            if constexpr (MSUM) {
#pragma unroll
                for (int u = 0; u < PVSTEPS; ++u) lacc = mfma16_bf16(sum_sel, pb[u], lacc);
            }
#pragma unroll
            for (int u = 0; u < PVSTEPS; ++u)
#pragma unroll
                for (int xb = 0; xb < XB; ++xb) {
                    u32x4_t a;
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int row = 16 * u + 4 * r + tr_row;
                        const int off = row * ROW_BYTES + (((4 * xb + tr_chunk) ^ v_swz<D>(row)) * 16) + tr_byte;
                        const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off));
                        const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
                        a[2 * r] = t2[0];
                        a[2 * r + 1] = t2[1];
                    }
                    if constexpr (D == 256) mma_o_a(oacc[xb], a, pb[u]);
                    else oacc[xb] = mfma_bf16(a, pb[u], oacc[xb]);
                }
            // Operand reads run pf_pv<D>() products ahead of the matrix cores; the
            // row-sum products, whose operands are already in registers, go
            // first while those reads are in flight.
            constexpr int NP = PVSTEPS * XB;
#pragma unroll
            for (int i = 0; i < pf_pv<D>(); ++i) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if constexpr (MSUM) __builtin_amdgcn_sched_group_barrier(0x008, PVSTEPS, 0);
#pragma unroll
            for (int i = 0; i < NP - pf_pv<D>(); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int i = 0; i < pf_pv<D>(); ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
        const bool sc = j < n && visible(j);
        if (sc && D == 256) {
            s_ring((const char *)(kcur + so), ic<LD>(), jl, knext, vnext);
        } else if (D != 256 && sc) {
            if constexpr (LD) { issue_v(jl, vnext); issue_k(jl, knext); }
            const char *ks = (const char *)(kcur + so);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
                const int row = kb * 32 + krow;
                const char *kr = ks + row * ROW_BYTES;
                const int sw = k_swz<D>(row);
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    const u32x4_t a = *(const u32x4_t *)(kr + (((2 * t + hf) ^ sw) * 16));
                    sacc[kb] = mfma_bf16(a, qreg[t], sacc[kb]);
                }
            }
            // the phase's 2*BPL loads go evenly after the product / operand-read pairs
            constexpr int NS = NKB * KSTEPS, NIT = NS - pf_qk<D>(), NL = 2 * BPL;
#pragma unroll
            for (int i = 0; i < pf_qk<D>(); ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int i = 0; i < NIT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int r = 0; r < NL; ++r)
                    if (LD && r * NIT / NL == i) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < pf_qk<D>(); ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        } else if constexpr (LD) {
            issue_v(jl, vnext);
            issue_k(jl, knext);
        }
    };

    // Reference-maximum update for a tile whose raw row maximum is mx, with
    // the accumulator rescale; returns the factor for the running sums.
    auto settle = [&](float mx) __attribute__((always_inline)) -> float {
        const float m_tile = mx * c;
        const bool grow = m_tile > m_run + kLazyLog2;
        float alpha = 1.f;
        if (grow) {
            alpha = __builtin_amdgcn_exp2f(m_run - m_tile);   // 0 on the first visit
            m_run = m_tile;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            sync_acc();
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[xb][i] *= alpha;
                if constexpr (D == 256) asm volatile("s_nop 3" : "+a"(oacc[xb]));
            }
            if constexpr (MSUM) {
#pragma unroll
                for (int i = 0; i < 4; ++i) lacc[i] *= alpha;
            }
        }
        return alpha;
    };
    auto tile_max = [&]() __attribute__((always_inline)) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        return max_halves(mx);
    };
    // P = 2^(s*c - m) rounded to bf16 and packed as the next product's B
    // operand; returns the fp32 row sum of the unrounded values.  The sums
    // start from the first pair (adding +0 first would cost an instruction:
    // it is not folded, for the sake of -0, which exp2 never returns).
    auto exps = [&]() __attribute__((always_inline)) -> float {
        const float m_sub = m_run == -INFINITY ? 0.f : m_run;
        float rf0 = 0.f, rf1 = 0.f;
#pragma unroll
        for (int u = 0; u < PVSTEPS; ++u) {
            const int kb = u >> 1, base = (u & 1) * 8;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][base + 2 * w], c, -m_sub));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][base + 2 * w + 1], c, -m_sub));
                rf0 = (u == 0 && w == 0) ? e0 : rf0 + e0;
                rf1 = (u == 0 && w == 0) ? e1 : rf1 + e1;
                pb[u][w] = pack_bf16(e0, e1);
            }
        }
        return rf0 + rf1;
    };

    // Vector-ALU step for tile j: mask (tiles crossing the diagonal or the
    // end only), the probabilities against the reference maximum, and both
    // row sums: fp32 over the unrounded values (the log-sum-exp), and over the
    // bf16 values the product consumes, which normalises O so that O stays a
    // convex combination of the V rows (on the matrix cores for d <= 128, see
    // lacc; at d = 256 two per v_dot2_f32_bf16 against (1, 1)).  The reference maximum is set from the exact maximum of the
    // first tile only; later tiles are exponentiated against it directly,
    // since any reference gives the same softmax (second page, section 5.1).
    // Should a row's scores run more than 64 (base 2) above the reference,
    // its tile sum exceeds 2^64 (or overflows), and that tile is redone with
    // its own maximum and the usual rescale.
    bool ref_set = false;      // block-sparse: the wavefront has set its reference (uniform)
    auto softmax_step = [&](int j) __attribute__((always_inline)) {
        if (!visible(j)) return;
        const int key0 = key_lo + tix(j) * kBN;
        const bool need_mask = (key0 + kBN > Nk) || (CAUSAL && key0 + kBN - 1 > wq0 + off);
        if (need_mask) {
            const int lim = (CAUSAL ? min(my_q + off, Nk - 1) : Nk - 1) - (key0 + 8 * hf);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb * 32 + 16 * (i >> 3) + (i & 7) > lim) sacc[kb][i] = -INFINITY;
        }
        float alpha = 1.f;
        // The reference comes from the exact maximum of the wavefront's first
        // visible tile (tile 0 without a block mask).  Every row that sees
        // any key sees one there: with a block mask all rows of a wavefront
        // share the mask row, and a row that the causal rule leaves empty in
        // that tile sees only larger keys, all masked, in later ones.
        if (SPARSE ? !ref_set : j == 0) {
            alpha = settle(tile_max());
            ref_set = true;
        }
        float rf = exps();
        if (__builtin_amdgcn_ballot_w64(rf > kFarSum) != 0) {
            alpha *= settle(tile_max());
            rf = exps();
        }
        l_run = l_run * alpha + rf;
        if constexpr (!MSUM) {
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int u = 0; u < PVSTEPS; ++u) {
                rs0 = sum_bf16x2(pb[u][0], rs0);
                rs1 = sum_bf16x2(pb[u][1], rs1);
                rs0 = sum_bf16x2(pb[u][2], rs0);
                rs1 = sum_bf16x2(pb[u][3], rs1);
            }
            lb_run = lb_run * alpha + (rs0 + rs1);
        }
    };

    // ---- ping-pong schedule.  Global phase t = 0 .. 2n+1.  A wavefront of
    // group g runs local step s = t - g: even s = 2j is the matrix-core step
    // for tile j, odd s = 2j+1 the vector-ALU step for tile j.  Group 1
    // trails group 0 by one phase, so on every SIMD one wavefront issues
    // matrix-core work while the other runs the softmax.  K_j and V_{j-1} are
    // read in phases 2j and 2j+1; K_{j+1} and V_j are loaded during those two
    // phases into the other stage.  The only barrier is the one after each odd
    // phase, which the stage swap needs.  Within a tile each wavefront moves
    // from its first step to its second as soon as it is done: the two
    // wavefronts of a SIMD still alternate, and neither waits for the slower
    // wavefronts of the other SIMDs halfway through the tile.
    if (n > 0) load_k(0, Ks0);
    lds_wait_vm();
    // The same wait as a builtin, which the compiler's own wait tracking
    // sees: the Q^T loads are then known to be complete inside the loop.
    // Otherwise it may put partial vmcnt waits for them before the first
    // products of a phase, and those would also wait for tile loads it does
    // not see (the inline-assembly ones).
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0), expcnt and lgkmcnt unconstrained
    finish_q();
    __syncthreads();
    const int nphase = 2 * n_loop + 2;    // the same on every wavefront: barriers match
    // G: the wavefront's group; P: the parity of global phase t (both
    // compile-time, so that each group's loop is straight-line code with its
    // loads in the same scheduling regions as its products).
    auto phase = [&](auto G, auto P, int t, const uint16_t *kcur, const uint16_t *vprev, uint16_t *knext,
                     uint16_t *vnext) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value, par = decltype(P)::value;
        // Even phases load K_{j+1} and V_j (j = t/2): with a block mask at the
        // start of the phase, otherwise spread through the leading group's
        // products.
        if constexpr (!SPREAD && !kSingleStage && par == 0) {
            const int j = t >> 1;
            if (j + 1 < n) load_k(j + 1, knext);
            if (j < n) load_v(j, vnext);
        }
        constexpr bool LD = SPREAD && !kSingleStage && par == 0 && g == 0;
        constexpr bool MSTEP = ((par - g) & 1) == 0;   // local step s = t - g is even
        const int s = t - g;
        if (s >= 0 && s <= 2 * n) {
            if constexpr (MSTEP) {
                // Matrix-core phases issue first when both wavefronts of a SIMD are ready.
                __builtin_amdgcn_s_setprio(1);
                mfma_step(ic<LD>(), s >> 1, kcur, vprev, t >> 1, knext, vnext);
                __builtin_amdgcn_s_setprio(0);
            } else {
                softmax_step(s >> 1);
            }
        } else if constexpr (LD) {
            issue_v(t >> 1, vnext);
            issue_k(t >> 1, knext);
        }
        if constexpr (par == 1) {            // K_{j+1}, V_j resident before phase 2j+2
            lds_wait_vm();
            __syncthreads();
        } else if constexpr (D == 64) {
            // d = 64 (half the products per softmax): a barrier after the even
            // phases too keeps the two groups aligned (measured +3%; at d = 128
            // it costs 2%).  It waits for LDS accesses only, not for the tile
            // loads still in flight.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };
    auto run = [&](auto G) __attribute__((always_inline)) {
        if constexpr (kSingleStage) {
            for (int t = 0; t < nphase; t += 2) {
                // The barrier after phase t - 1 ended every read of the stage
                // (K_0 was loaded before the loop).
                const int j = t >> 1;
                if (j >= 1) {
                    if (j < n) load_k(j, Ks0);
                    if (j - 1 < n) load_v(j - 1, Vs0);
                    lds_wait_vm();
                    __syncthreads();
                }
                phase(G, ic<0>(), t, Ks0, Vs0, Ks1, Vs1);
                phase(G, ic<1>(), t + 1, Ks0, Vs0, Ks1, Vs1);
            }
            return;
        }
        for (int t = 0; t < nphase; t += 4) {
            // even j = t/2: K_j in Ks0, V_{j-1} in Vs1; loads go to Ks1, Vs0
            phase(G, ic<0>(), t, Ks0, Vs1, Ks1, Vs0);
            phase(G, ic<1>(), t + 1, Ks0, Vs1, Ks1, Vs0);
            if (t + 2 < nphase) {
                // odd j: K_j in Ks1, V_{j-1} in Vs0; loads go to Ks0, Vs1
                phase(G, ic<0>(), t + 2, Ks1, Vs0, Ks0, Vs1);
                phase(G, ic<1>(), t + 3, Ks1, Vs0, Ks0, Vs1);
            }
        }
    };
    if constexpr (NWAVES == 8) {
        if (grp == 0) run(ic<0>());
        else run(ic<1>());
    } else {
        run(ic<0>());
    }

    sync_acc();
    // ---- epilogue: O = O_acc / l (bf16, round to nearest even), lse = m ln2 + ln l.
    // A row that saw no key (l = 0) gets O = 0 and lse = -inf.  A split
    // forward stores O in fp32 and the log-sum-exp of its key range instead.
    const float l_tot = sum_halves(l_run);
    const float lb_tot = MSUM ? lacc[0] : sum_halves(lb_run);
    if (my_q < Nq) {
        const bool empty = l_tot == 0.f;
        const float inv = empty ? 0.f : 1.f / lb_tot;
        const float lse_row = empty ? -INFINITY : m_run * kLn2 + logf(l_tot);
        const int64_t row = ((int64_t)split * p.B + b) * p.Hq + h;   // split = 0 unless SPLIT
        if (SPLIT) {
            float *orow = p.o_part + (row * Nq + my_q) * D;
#pragma unroll
            for (int xb = 0; xb < XB; ++xb)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int x = xb * 32 + 8 * gi + 4 * hf;
                    const f32x4_t w = {oacc[xb][4 * gi] * inv, oacc[xb][4 * gi + 1] * inv,
                                       oacc[xb][4 * gi + 2] * inv, oacc[xb][4 * gi + 3] * inv};
                    *(f32x4_t *)(orow + x) = w;
                }
            if (hf == 0) p.lse_part[row * Nq + my_q] = lse_row;
        } else {
            uint16_t *orow = (uint16_t *)p.o + ((int64_t)b * Nq * p.Hq + h) * D + (int64_t)my_q * sQ;
#pragma unroll
            for (int xb = 0; xb < XB; ++xb)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int x = xb * 32 + 8 * gi + 4 * hf;
                    u32x2_t w = {pack_bf16(oacc[xb][4 * gi] * inv, oacc[xb][4 * gi + 1] * inv),
                                 pack_bf16(oacc[xb][4 * gi + 2] * inv, oacc[xb][4 * gi + 3] * inv)};
                    *(u32x2_t *)(orow + x) = w;
                }
            if (hf == 0) p.lse[row * Nq + my_q] = lse_row;
        }
    }
}

template <int D, bool CAUSAL, bool SPLIT, bool SPARSE>
hipError_t launch_one(const FwdParams &p_in, hipStream_t stream)
{
    FwdParams p = p_in;
    p.ntiles = (p.Nq + wg_rows<D>() - 1) / wg_rows<D>();
    const unsigned grid = (unsigned)p.B * (unsigned)p.Hq * (unsigned)p.ntiles * (unsigned)p.nsplit;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, SPLIT, SPARSE>), dim3(grid), dim3(wg_threads<D>()), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams &p, hipStream_t stream)
{
    if (p.block_mask)
        return p.causal ? launch_one<D, true, false, true>(p, stream) : launch_one<D, false, false, true>(p, stream);
    if (p.nsplit > 1)
        return p.causal ? launch_one<D, true, true, false>(p, stream) : launch_one<D, false, true, false>(p, stream);
    return p.causal ? launch_one<D, true, false, false>(p, stream) : launch_one<D, false, false, false>(p, stream);
}

}  // namespace

int fwd_bf16_lds_stages() { return kSingleStage ? 1 : 2; }

hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t stream)
{
    if (d == 256) return launch_d<256>(p, stream);
    return d == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace fa
