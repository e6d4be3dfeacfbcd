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
// One thread handles four consecutive elements of one row; the D/4 threads
// of a row read its partials as contiguous float4s, and rows are taken in
// the (batch, head, query) order of the partial buffers.
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
__global__ void __launch_bounds__(kThreads) combine_kernel(FwdParams p)
{
    constexpr int TPR = D / 4;              // threads per row
    constexpr int RPB = kThreads / TPR;     // rows per workgroup
    const int tid = threadIdx.x;
    const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    const int x = (tid % TPR) * 4;
    if (row >= rows) return;

    float mx = -INFINITY;
    for (int r = 0; r < p.nsplit; ++r) mx = fmaxf(mx, p.lse_part[r * rows + row]);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != -INFINITY) {
        for (int r = 0; r < p.nsplit; ++r) {
            const float lr = p.lse_part[r * rows + row];
            if (lr == -INFINITY) continue;
            const float w = expf(lr - mx);
            wsum += w;
            acc += w * *(const f32x4_t *)(p.o_part + (r * rows + row) * D + x);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
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
    if (x == 0) p.lse[row] = mx == -INFINITY ? -INFINITY : mx + logf(wsum);
}

template <int D, bool OUT_BF16>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    constexpr int RPB = kThreads / (D / 4);
    const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
    const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((combine_kernel<D, OUT_BF16>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const FwdParams &p, int d, int out_bf16, hipStream_t stream)
{
    if (d == 128) return out_bf16 ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return out_bf16 ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace fa
