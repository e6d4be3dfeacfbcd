// Merge of the partial results of a split-key forward.
//
// Each key range r of a query row produced a normalised partial output O_r
// (the softmax over that range alone, applied to its V rows) and the
// log-sum-exp L_r of its scaled scores (-inf when the range held no key the
// row can see).  The full row follows from the same rescaling the online
// softmax uses between blocks ("FlashAttention：IO 感知的精确注意力",
// section 5, and its section 12.1 for the decode use, where the key sequence
// is split so that its parts run in parallel):
//     M = max_r L_r,  w_r = exp(L_r - M),  O = sum_r w_r O_r / sum_r w_r,
//     lse = M + ln(sum_r w_r).
// A row for which every range is empty keeps O = 0 and lse = -inf.
//
// A row's D/4 threads each own four consecutive elements (one float4), and
// `spl` such thread groups split the ranges of the row between them (range
// r goes to group r % spl), so that rows with many ranges (decoding) still
// spread their loads over many threads.  Each group merges its ranges in one
// pass with a running maximum (the same rescaling again), so all of its
// loads can be in flight at once; the groups' results are then merged
// through LDS.  A workgroup holds 256 / (D/4 * spl) rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) combine_kernel(FwdParams p, int spl)
{
    constexpr int TPR = D / 4;                   // threads per row and range group
    const int tid = threadIdx.x;
    const int chunk = tid % TPR;
    const int sl = (tid / TPR) % spl;            // range group
    const int rloc = tid / (TPR * spl);          // row within the workgroup
    const int rpb = kThreads / (TPR * spl);
    const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
    const int64_t row = (int64_t)blockIdx.x * rpb + rloc;
    const bool live = row < rows;
    const int x = chunk * 4;

    __shared__ float red_m[kThreads / 16];                   // [row][group]; spl * rpb <= 256 / 16
    __shared__ float red_w[kThreads / 16];
    __shared__ __attribute__((aligned(16))) f32x4_t red_o[kThreads];

    // this group's ranges, four at a time while four remain (the loads of a
    // batch are issued together), then one at a time; each is merged against
    // the running maximum m without branches.  An empty range (L_r = -inf)
    // gets weight 0, and while every range so far was empty (m = -inf)
    // nothing is rescaled.
    float m = -INFINITY, wsum = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto merge = [&](float l, f32x4_t o) {
        const float m_new = fmaxf(m, l);
        const float a = m_new == -INFINITY ? 1.f : expf(m - m_new);   // 0 when m is -inf
        const float w = l == -INFINITY ? 0.f : expf(l - m_new);
        acc = acc * a + w * o;
        wsum = wsum * a + w;
        m = m_new;
    };
    if (live) {
        int r = sl;
        for (; r + 3 * spl < p.nsplit; r += 4 * spl) {
            float lr[4];
            f32x4_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lr[k] = p.lse_part[(r + k * spl) * rows + row];
                o[k] = *(const f32x4_t *)(p.o_part + ((r + k * spl) * rows + row) * D + x);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) merge(lr[k], o[k]);
        }
        for (; r < p.nsplit; r += spl)
            merge(p.lse_part[r * rows + row], *(const f32x4_t *)(p.o_part + (r * rows + row) * D + x));
    }
    red_o[tid] = acc;
    if (chunk == 0) {
        red_m[rloc * spl + sl] = m;
        red_w[rloc * spl + sl] = wsum;
    }
    __syncthreads();
    if (sl != 0 || !live) return;
    float M = -INFINITY;
    for (int j = 0; j < spl; ++j) M = fmaxf(M, red_m[rloc * spl + j]);
    float W = 0.f;
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int j = 0; j < spl; ++j) {
            const float mj = red_m[rloc * spl + j];
            if (mj == -INFINITY) continue;
            const float a = expf(mj - M);
            W += a * red_w[rloc * spl + j];
            acc += a * red_o[tid + j * TPR];
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    acc *= inv;

    // row = (b * Hq + h) * Nq + i; o is [B][Nq][Hq][D], lse is [B][Hq][Nq]
    const int64_t bh = row / p.Nq;
    const int i = (int)(row - bh * p.Nq);
    const int b = (int)(bh / p.Hq), h = (int)(bh - (int64_t)b * p.Hq);
    const int64_t o_off = (((int64_t)b * p.Nq + i) * p.Hq + h) * D + x;
    if (OUT_BF16) {
        const u32x2_t w = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
        *(u32x2_t *)((uint16_t *)p.o + o_off) = w;
    } else {
        *(f32x4_t *)((float *)p.o + o_off) = acc;
    }
    if (chunk == 0) p.lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
}

template <int D, bool OUT_BF16>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    constexpr int TPR = D / 4;
    int spl = 1;                                  // range groups: a power of two, at most the ranges
    while (spl < p.nsplit && spl * 2 * TPR <= kThreads) spl *= 2;
    const int rpb = kThreads / (TPR * spl);
    const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
    const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
    hipLaunchKernelGGL((combine_kernel<D, OUT_BF16>), dim3(grid), dim3(kThreads), 0, stream, p, spl);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const FwdParams &p, int d, int out_bf16, hipStream_t stream)
{
    if (d == 256) return out_bf16 ? launch_one<256, true>(p, stream) : launch_one<256, false>(p, stream);
    if (d == 128) return out_bf16 ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return out_bf16 ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace fa
