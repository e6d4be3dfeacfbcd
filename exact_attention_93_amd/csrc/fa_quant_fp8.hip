// Block-scaled e4m3 quantisation of a bf16 [B][N][H][d] tensor (d = 128), with
// optional incoherent processing, for the fp8 forward with per-block scales.
//
// The second page ("FlashAttention：IO 感知的精确注意力", section 10, the FP8
// lever of FlashAttention-3, and section 12.2) credits two measures with
// keeping FP8 attention accurate: one scale per block instead of one per
// tensor, and incoherent processing, which rotates the vectors so that an
// outlier coordinate is spread over all of them before quantisation.
//
// Here a block is 64 consecutive rows of one head (all d coordinates) and its
// scale a power of two 2^e, the form the gfx950 scaled fp8 products apply for
// free; e is the smallest integer with max|y| / 2^e <= 448 (the largest e4m3
// value), -127 for a block of zeros, and each element is stored as the e4m3
// code nearest to y / 2^e (ties to even; v_cvt_pk_fp8_f32).  With a sign
// vector s, y = (x * s) H, H the d x d Sylvester-Hadamard matrix, computed in
// fp32 by the radix-2 butterfly network in stage order h = 1, 2, ..., 64:
// rotating q and k alike multiplies every score by d exactly.
//
// Work partition: one workgroup of 256 threads per (block, head, batch).  A
// row is held by 16 lanes, 8 coordinates each (lane i: 8i .. 8i+7), so the
// butterfly stages h = 1, 2, 4 stay inside a lane and h = 8 .. 64 exchange
// with lane i ^ (h / 8).  Each wavefront takes 16 rows, 4 at a time; the
// rotated values stay in registers while the block maximum is reduced
// (in-wavefront shuffles, then LDS over the 4 wavefronts), then are scaled,
// converted and stored.  The kernel reads and writes every byte once, so HBM
// bandwidth bounds it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int kRows = kQuantBlock;           // rows per block
constexpr int kThreads = 256;
constexpr int kRowsPerIter = kThreads / 16;  // 16 rows of the block per pass (4 per wavefront)
constexpr int kIters = kRows / kRowsPerIter;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Smallest e with amax / 2^e <= 448, from the bits of amax (amax = m 2^E,
// 1 <= m < 2, and 448 = 1.75 2^8): e = E - 8, plus 1 when m > 1.75.
__device__ __forceinline__ int block_exponent(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    const int field = (int)(u >> 23);
    if (field == 0) return -127;                     // zero or subnormal: far below any e4m3 step
    const int E = field - 127;
    const uint32_t mant = u & 0x7fffffu;
    int e = E - 8 + (mant > 0x600000u ? 1 : 0);      // 1.75 = 1 + 0x600000 / 2^23
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__global__ void __launch_bounds__(kThreads) quant_fp8_kernel(QuantParams p)
{
    const int nb = (p.N + kRows - 1) / kRows;
    const int blk = blockIdx.x % nb;
    const int bh = blockIdx.x / nb;
    const int h = bh % p.H, b = bh / p.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15;                        // 8 coordinates: 8*li .. 8*li+7
    const int rsub = lane >> 4;                      // row within the wavefront's 4
    const int64_t row_stride = (int64_t)p.H * D;     // elements between consecutive rows
    const int64_t base = ((int64_t)b * p.N) * row_stride + (int64_t)h * D + 8 * li;

    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 1.f;
    if (p.signs) {
        const uint64_t w = *(const uint64_t *)(p.signs + 8 * li);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = (int8_t)(w >> (8 * e)) < 0 ? -1.f : 1.f;
    }

    float y[kIters][8];
    float amax = 0.f;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int row = blk * kRows + it * kRowsPerIter + wave * 4 + rsub;
        float x[8];
        if (row < p.N) {
            const u32x4_t v = *(const u32x4_t *)((const uint16_t *)p.x + base + row * row_stride);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_to_f32(v[e] & 0xffffu);
                x[2 * e + 1] = bf16_to_f32(v[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        if (p.signs) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= s[e];
            // stages h = 1, 2, 4 inside the lane
#pragma unroll
            for (int hh = 1; hh < 8; hh *= 2)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!(e & hh)) {
                        const float a = x[e], c = x[e + hh];
                        x[e] = a + c;
                        x[e + hh] = a - c;
                    }
            // stages h = 8 .. 64: partner lane li ^ (h / 8); the lane holding
            // the lower index keeps a + b, the other a - b (a lower, b upper)
#pragma unroll
            for (int m = 1; m < 16; m *= 2) {
                const bool upper = (li & m) != 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float other = __shfl_xor(x[e], m, 64);
                    x[e] = upper ? other - x[e] : x[e] + other;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[it][e] = x[e];
            amax = fmaxf(amax, fabsf(x[e]));
        }
    }
    // block maximum: wavefront, then the four wavefronts through LDS
#pragma unroll
    for (int m = 1; m < 64; m *= 2) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    __shared__ float wmax[kThreads / 64];
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const int e = block_exponent(amax);
    if (threadIdx.x == 0) p.exps[(int64_t)bh * nb + blk] = (int8_t)e;
    // y / 2^e exactly (a power of two; the result is at most 448)
    const float inv = __builtin_ldexpf(1.f, -e);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int row = blk * kRows + it * kRowsPerIter + wave * 4 + rsub;
        if (row >= p.N) continue;
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[it][0] * inv, y[it][1] * inv, 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[it][2] * inv, y[it][3] * inv, w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[it][4] * inv, y[it][5] * inv, 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[it][6] * inv, y[it][7] * inv, w1, true);
        *(u32x2_t *)((uint8_t *)p.codes + base + row * row_stride) = u32x2_t{(uint32_t)w0, (uint32_t)w1};
    }
}

}  // namespace

hipError_t launch_quant_fp8(const QuantParams &p, hipStream_t stream)
{
    const int nb = (p.N + kRows - 1) / kRows;
    const unsigned grid = (unsigned)p.B * (unsigned)p.H * (unsigned)nb;
    hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
