// Fused exact attention forward, bf16 in / bf16 out, fp32 accumulation, for
// CDNA4 (gfx950) matrix cores.
//
// Algorithm: the Q-block-outer loop of FlashAttention-2 ("[Attention优化]
// 从Online-Softmax到FlashAttention V1/V2/V3", section 0x05; "Flash-attention
// 学习", section 2.2): a workgroup owns 128 query rows of one (batch, head),
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
// Work partition inside the workgroup: four wavefronts share each K/V tile
// and each owns 32 whole query rows, so row statistics never cross
// wavefronts (the "sliced-Q" partition the pages credit to FlashAttention-2).
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, D = A*B + C, 32x32 output):
// the kernel computes the TRANSPOSED score tile S^T = K Q^T (A = K from LDS,
// B = Q^T from registers).  A 32x32 accumulator holds column (lane % 32) in
// every lane, so lane l owns query (l % 32) and 16 of the 32 keys of a block;
// the other 16 are in lane l ^ 32.  A row maximum or sum is therefore 16
// in-lane operations plus one exchange between the two lane halves.  The K
// rows are fed to the A operand in a permuted order (bits 2 and 3 of the row
// index swapped) so that accumulator register i of lane half hf holds key
// 16*(i/8) + 8*hf + (i%8): exactly the slots the B operand of the next
// product expects.  The probabilities then feed O^T = V^T P^T straight from
// registers (B = P^T, A = V^T from LDS), and the O^T accumulator again has
// one query per lane, so the rescale by exp(m_old - m_new) is a per-lane
// scalar.  V is written to LDS transposed ([d][key]) so that each A-operand
// fetch is one 16-byte read.
//
// Exponentials are taken base 2 with scale*log2(e) folded into one FMA per
// score.  The accumulator is only rescaled when some row's maximum grows by
// more than kLazyLog2 (base-2 units) over the reference value in use: the
// result does not depend on which reference value is subtracted ("the
// softmax identity holds for any m", second page, section 5.1), the values
// stay bounded by 2^kLazyLog2, and the final division uses the same l.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = kBlockM;   // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;  // 4 wavefronts of 64
constexpr float kLazyLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
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

__device__ __forceinline__ float other_half(float x)
{
    return __shfl_xor(x, 32);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) fwd_bf16_kernel(FwdParams p)
{
    constexpr int KSTEPS = D / 16;                 // K-steps of S^T = K Q^T
    constexpr int XB = D / 32;                     // 32-row blocks of O^T
    constexpr int NKB = kBN / 32;                  // 32-key blocks per tile
    constexpr int PVSTEPS = kBN / 16;              // K-steps of O^T = V^T P^T
    constexpr int KCH = D / 8;                     // 16-byte chunks per row
    constexpr int RPP = kThreads / KCH;            // rows per load pass
    constexpr int LOADS = kBN / RPP;               // 16-byte loads per thread per tensor
    constexpr int VT_PITCH = kBN + 8;              // V^T row pitch (elements)
    static_assert(LOADS == 2 || LOADS == 4, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VT_PITCH];

    int b, h, tile;
    decode_tile(p, b, h, tile);
    const int hk = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hf = lane >> 5;
    const int N = p.N;
    const int q_first = tile * kBM;
    const int wq0 = q_first + wave * 32;          // first query row of this wavefront
    const int my_q = wq0 + lq;                    // query row owned by this lane
    const float c = p.c;

    const int sQ = p.Hq * D, sK = p.Hkv * D;      // row strides (elements)
    const uint16_t *qbase = (const uint16_t *)p.q + ((int64_t)b * N * p.Hq + h) * D;
    const uint16_t *kbase = (const uint16_t *)p.k + ((int64_t)b * N * p.Hkv + hk) * D;
    const uint16_t *vbase = (const uint16_t *)p.v + ((int64_t)b * N * p.Hkv + hk) * D;

    // ---- Q^T operand: lane (lq, hf) holds q[my_q][16t + 8hf .. +7] for step t
    u32x4_t qreg[KSTEPS];
    if (my_q < N) {
        const u32x4_t *src = (const u32x4_t *)(qbase + my_q * sQ);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = src[2 * t + hf];
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = u32x4_t{0, 0, 0, 0};
    }
    if (p.qmode != 0) {
        const uint32_t keep = p.qmode == 2 ? 0u : 0xffffffffu;
        const uint32_t flip = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[t][e] = (qreg[t][e] ^ flip) & keep;
    }

    // ---- number of K/V tiles this workgroup visits
    int nkt = (N + kBN - 1) / kBN;
    if (CAUSAL) {
        const int last_q = min(q_first + kBM, N) - 1;
        nkt = last_q / kBN + 1;
    }

    // ---- global -> register staging of one K/V tile
    const int ch = tid % KCH;      // 16-byte chunk of a row this thread moves
    const int rg = tid / KCH;      // row (K) / key group (V) this thread moves
    u32x4_t kst[LOADS], vst[LOADS];
    auto gload = [&](int j) {
        const int key0 = j * kBN;
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int key = key0 + rg + r * RPP;
            kst[r] = key < N ? *(const u32x4_t *)(kbase + key * sK + ch * 8) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int key = key0 + rg * LOADS + r;
            vst[r] = key < N ? *(const u32x4_t *)(vbase + key * sK + ch * 8) : u32x4_t{0, 0, 0, 0};
        }
    };
    // register -> LDS: K row-major with the 16-byte chunk index XOR-swizzled by
    // the row; V transposed to [d][key].
    auto lstore = [&](int buf) {
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int row = rg + r * RPP;
            *(u32x4_t *)&Ks[buf][row * D + ((ch ^ (row & (KCH - 1))) * 8)] = kst[r];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {          // dword w holds x = 2w (low) and 2w+1 (high)
            const int x = ch * 8 + 2 * w;
            if constexpr (LOADS == 4) {
                const uint32_t a0 = vst[0][w], a1 = vst[1][w], a2 = vst[2][w], a3 = vst[3][w];
                const u32x2_t ev = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
                const u32x2_t od = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
                *(u32x2_t *)&Vt[buf][x * VT_PITCH + rg * 4] = ev;
                *(u32x2_t *)&Vt[buf][(x + 1) * VT_PITCH + rg * 4] = od;
            } else {
                const uint32_t a0 = vst[0][w], a1 = vst[1][w];
                *(uint32_t *)&Vt[buf][x * VT_PITCH + rg * 2] = (a0 & 0xffffu) | (a1 << 16);
                *(uint32_t *)&Vt[buf][(x + 1) * VT_PITCH + rg * 2] = (a0 >> 16) | (a1 & 0xffff0000u);
            }
        }
    };

    // A-operand row for lane lq: key 32*kb + perm(lq), perm swaps bits 2 and 3.
    const int krow = (lq & 0x13) | ((lq & 4) << 1) | ((lq & 8) >> 1);

    float m_run = -INFINITY;   // reference maximum (base-2 units), shared by both halves
    float l_run = 0.f;         // fp32 sum of this lane half's probabilities
    float lb_run = 0.f;        // the same sum over their bf16-rounded values
    f32x16_t oacc[XB];
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[xb][i] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < nkt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nkt) gload(j + 1);
        const uint16_t *ks = Ks[buf];
        const uint16_t *vt = Vt[buf];
        const int key0 = j * kBN;
        const bool active = !CAUSAL || key0 <= wq0 + 31;   // some key visible to this wave
        if (active) {
            // ---- S^T = K Q^T
            f32x16_t sacc[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
                const int row = kb * 32 + krow;
                const uint16_t *kr = ks + row * D;
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    const u32x4_t a = *(const u32x4_t *)(kr + (((2 * t + hf) ^ (row & (KCH - 1))) * 8));
                    sacc[kb] = mfma_bf16(a, qreg[t], sacc[kb]);
                }
            }
            // ---- mask: keys past the end, and keys after the query when causal
            const bool need_mask = (key0 + kBN > N) || (CAUSAL && key0 + kBN - 1 > wq0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + kb * 32 + 16 * (i >> 3) + 8 * hf + (i & 7);
                        const bool vis = key < N && (!CAUSAL || key <= my_q);
                        if (!vis) sacc[kb][i] = -INFINITY;
                    }
            }
            // ---- row maximum of this tile (16 in-lane values per block + one exchange)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
            mx = fmaxf(mx, other_half(mx));
            const float m_tile = mx * c;
            const bool grow = m_tile > m_run + kLazyLog2;
            float alpha = 1.f;
            if (grow) {
                alpha = __builtin_amdgcn_exp2f(m_run - m_tile);   // 0 on the first visit
                m_run = m_tile;
            }
            const float m_sub = m_run == -INFINITY ? 0.f : m_run;
            // ---- P = 2^(s*c - m); fp32 row sum (for the log-sum-exp)
            float rf0 = 0.f, rf1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    sacc[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c, -m_sub));
                    sacc[kb][i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i + 1], c, -m_sub));
                    rf0 += sacc[kb][i];
                    rf1 += sacc[kb][i + 1];
                }
            l_run = l_run * alpha + (rf0 + rf1);
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int xb = 0; xb < XB; ++xb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[xb][i] *= alpha;
            }
            // ---- O^T += V^T P^T.  A second row sum is taken over the same
            // bf16-rounded probabilities the product consumes (two per
            // v_dot2_f32_bf16 against (1, 1)) and normalises O, so that
            // O = sum p v / sum p stays a convex combination of the V rows;
            // the fp32 sum above gives the log-sum-exp.
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int u = 0; u < PVSTEPS; ++u) {
                const int kb = u >> 1, base = (u & 1) * 8;
                u32x4_t pb;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pb[w] = pack_bf16(sacc[kb][base + 2 * w], sacc[kb][base + 2 * w + 1]);
                rs0 = sum_bf16x2(pb[0], rs0);
                rs1 = sum_bf16x2(pb[1], rs1);
                rs0 = sum_bf16x2(pb[2], rs0);
                rs1 = sum_bf16x2(pb[3], rs1);
#pragma unroll
                for (int xb = 0; xb < XB; ++xb) {
                    const u32x4_t a = *(const u32x4_t *)(vt + (xb * 32 + lq) * VT_PITCH + 16 * u + 8 * hf);
                    oacc[xb] = mfma_bf16(a, pb, oacc[xb]);
                }
            }
            lb_run = lb_run * alpha + (rs0 + rs1);
        }
        if (j + 1 < nkt) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l (bf16, round to nearest even), lse = m ln2 + ln l
    const float l_tot = l_run + other_half(l_run);
    const float lb_tot = lb_run + other_half(lb_run);
    if (my_q < N) {
        const float inv = 1.f / lb_tot;
        uint16_t *orow = (uint16_t *)p.o + ((int64_t)b * N * p.Hq + h) * D + my_q * sQ;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int x = xb * 32 + 8 * gi + 4 * hf;
                u32x2_t w = {pack_bf16(oacc[xb][4 * gi] * inv, oacc[xb][4 * gi + 1] * inv),
                             pack_bf16(oacc[xb][4 * gi + 2] * inv, oacc[xb][4 * gi + 3] * inv)};
                *(u32x2_t *)(orow + x) = w;
            }
        if (hf == 0) p.lse[((int64_t)b * p.Hq + h) * N + my_q] = m_run * kLn2 + logf(l_tot);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    const unsigned grid = (unsigned)p.B * (unsigned)p.Hq * (unsigned)p.ntiles;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t stream)
{
    if (d == 128) return p.causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return p.causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace fa
