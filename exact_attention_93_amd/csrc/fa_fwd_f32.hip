// Fused exact attention forward with fp32 inputs, output and arithmetic, on
// the CDNA4 fp32 matrix-core instruction v_mfma_f32_32x32x2_f32.
//
// Same algorithm and work partition as the bf16 kernel (Q-block-outer loop,
// online-softmax merge with deferred normalisation, causal tiles above the
// diagonal skipped; see fa_fwd_bf16.hip for the citations), with 32-key
// tiles and V kept in its natural [key][d] layout.  Two LDS buffers: the
// next tile's loads go to registers while the current tile's products run,
// and into the other buffer after them, one barrier per tile.  The
// single-stage build (FA_SINGLE_STAGE) loads each tile into one buffer
// between two barriers instead; the arithmetic is the same.
//
// Layout (32x32x2 fp32 MFMA): A lane l supplies A[l % 32][l / 32], B lane l
// supplies B[l / 32][l % 32]; the 32x32 accumulator holds column l % 32 in
// lane l and row 8*(i/4) + 4*(l/32) + (i%4) in register i.  S^T = K Q^T puts
// query l % 32 in lane l; O^T = V^T P^T then takes P^T straight from the
// S^T registers, one key pair (register i of both lane halves) per step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = kBlockM;
constexpr int kBN = 32;
constexpr int kThreads = 256;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two wavefronts per SIMD (two workgroups per compute unit, 66.5 KB of LDS
// each): the register budget is 256 per wavefront, which the kernel meets
// without spilling (at d = 128, 249 VGPRs and the accumulators among them).
template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(kThreads, 2) fwd_f32_kernel(FwdParams p)
{
    constexpr int KP = D + 4;              // K row pitch (floats)
    constexpr int S4 = D / 8;              // float4 groups of Q per lane
    constexpr int XB = D / 32;
    constexpr int LOADS = kBN * D / 4 / kThreads;   // float4 loads per thread per tensor

    constexpr int NBUF = kSingleStage ? 1 : 2;
    __shared__ __attribute__((aligned(16))) float Ks[NBUF][kBN * KP];
    __shared__ __attribute__((aligned(16))) float Vs[NBUF][kBN * D];

    int b, h, tile, split;
    decode_tile(p, b, h, tile, split);
    const int hk = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hf = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = p.off;
    const int q_first = tile * kBM;
    const int wq0 = q_first + wave * 32;
    const int my_q = wq0 + lq;
    const float c = p.c;

    const int sQ = p.Hq * D, sK = p.Hkv * D;
    const float *qbase = (const float *)p.q + ((int64_t)b * Nq * p.Hq + h) * D;
    const float *kbase = (const float *)p.k + ((int64_t)b * Nk * p.Hkv + hk) * D;
    const float *vbase = (const float *)p.v + ((int64_t)b * Nk * p.Hkv + hk) * D;

    // Q^T operand: step (s, e) of the contraction uses d = 8s + 4hf + e.
    f32x4_t qreg[S4];
    const float qmul = p.qmode == 1 ? -1.f : 1.f;
#pragma unroll
    for (int s = 0; s < S4; ++s) {
        if (my_q < Nq && p.qmode != 2) qreg[s] = *(const f32x4_t *)(qbase + my_q * sQ + 8 * s + 4 * hf) * qmul;
        else qreg[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    int kt_lo, kt_hi;
    key_tiles<kBN>(p, q_first, kBM, split, kt_lo, kt_hi);

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[XB];
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[xb][i] = 0.f;

    // Tile j of K and V: global memory -> registers (fetch), registers ->
    // LDS buffer (store); keys at or past Nk read as zero.
    f32x4_t kreg[LOADS], vreg[LOADS];
    auto fetch = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int idx = tid + r * kThreads;          // float4 index within the tile
            const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const int key = j * kBN + row;
            kreg[r] = vreg[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (key < Nk) {
                kreg[r] = *(const f32x4_t *)(kbase + key * sK + col);
                vreg[r] = *(const f32x4_t *)(vbase + key * sK + col);
            }
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int idx = tid + r * kThreads;
            const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
            *(f32x4_t *)&Ks[buf][row * KP + col] = kreg[r];
            *(f32x4_t *)&Vs[buf][row * D + col] = vreg[r];
        }
    };
    // The products and the softmax of tile j from LDS buffer buf.
    auto tile_step = [&](int j, int buf) __attribute__((always_inline)) {
        const int key0 = j * kBN;
        if (wq0 >= Nq || (CAUSAL && key0 > wq0 + 31 + off)) return;   // no row of this wave sees the tile
        const float *ks = Ks[buf];
        const float *vs = Vs[buf];

        f32x16_t sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < S4; ++s) {
            const f32x4_t a = *(const f32x4_t *)&ks[lq * KP + 8 * s + 4 * hf];
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc = mfma_f32(a[e], qreg[s][e], sacc);
        }
        if ((key0 + kBN > Nk) || (CAUSAL && key0 + kBN - 1 > wq0 + off)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (!(key < Nk && (!CAUSAL || key <= my_q + off))) sacc[i] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * c);
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_sub);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = exp2f(__builtin_fmaf(sacc[i], c, -m_sub));
            sacc[i] = e;
            rs = i == 0 ? e : rs + e;   // from the first value, not from +0
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[xb][i] *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
                oacc[xb] = mfma_f32(vs[key * D + xb * 32 + lq], sacc[i], oacc[xb]);
            }
        }
    };

    if constexpr (kSingleStage) {
        for (int j = kt_lo; j < kt_hi; ++j) {
            __syncthreads();   // previous tile fully consumed
            fetch(j);
            store(0);
            __syncthreads();
            tile_step(j, 0);
        }
    } else {
        if (kt_lo < kt_hi) {
            fetch(kt_lo);
            store(0);
        }
        __syncthreads();
        for (int j = kt_lo; j < kt_hi; ++j) {
            // Buffer buf holds tile j; the other was last read for tile j-1,
            // and the barrier that ended that tile ended those reads.
            const int buf = (j - kt_lo) & 1;
            const bool more = j + 1 < kt_hi;
            if (more) fetch(j + 1);
            tile_step(j, buf);
            if (more) store(buf ^ 1);
            __syncthreads();
        }
    }

    // A row that saw no key (l = 0) gets O = 0 and lse = -inf; a split
    // forward stores the result of its key range in the partial buffers.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (my_q < Nq) {
        const bool empty = l_tot == 0.f;
        const float inv = empty ? 0.f : 1.f / l_tot;
        const float lse_row = empty ? -INFINITY : m_run * kLn2 + logf(l_tot);
        const int64_t row = ((int64_t)split * p.B + b) * p.Hq + h;   // split = 0 unless SPLIT
        float *orow = SPLIT ? p.o_part + (row * Nq + my_q) * D
                            : (float *)p.o + ((int64_t)b * Nq * p.Hq + h) * D + (int64_t)my_q * sQ;
#pragma unroll
        for (int xb = 0; xb < XB; ++xb)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int x = xb * 32 + 8 * gi + 4 * hf;
                f32x4_t w = {oacc[xb][4 * gi] * inv, oacc[xb][4 * gi + 1] * inv,
                             oacc[xb][4 * gi + 2] * inv, oacc[xb][4 * gi + 3] * inv};
                *(f32x4_t *)(orow + x) = w;
            }
        if (hf == 0) (SPLIT ? p.lse_part : p.lse)[row * Nq + my_q] = lse_row;
    }
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    const unsigned grid = (unsigned)p.B * (unsigned)p.Hq * (unsigned)p.ntiles * (unsigned)p.nsplit;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, SPLIT>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams &p, hipStream_t stream)
{
    if (p.nsplit > 1)
        return p.causal ? launch_one<D, true, true>(p, stream) : launch_one<D, false, true>(p, stream);
    return p.causal ? launch_one<D, true, false>(p, stream) : launch_one<D, false, false>(p, stream);
}

}  // namespace

int fwd_f32_lds_stages() { return kSingleStage ? 1 : 2; }

hipError_t launch_fwd_f32(const FwdParams &p_in, int d, hipStream_t stream)
{
    FwdParams p = p_in;
    p.ntiles = (p.Nq + kBM - 1) / kBM;
    return d == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace fa
