// Attention forward for few query rows against many keys (decoding), bf16
// in, fp32 accumulation, on CDNA4 (gfx950) matrix cores.
//
// The decoding step of the second page's section 12.1 ("FlashAttention：IO
// 感知的精确注意力"): one (or a few) query rows per head meet a long key
// sequence, so batch x heads alone cannot fill the GPU and the keys are
// split into ranges that run in parallel; the ranges are merged afterwards
// with the online-softmax rescaling (fa_combine.hip).  The work is bound by
// reading K and V once from HBM, so the kernel is organised around that:
//
//  * All query rows that read the same key/value head (the group of query
//    heads of grouped-query attention, times the query rows) are packed
//    into the 32 rows of one matrix-core tile, so every K/V byte is fetched
//    once per group, not once per query head (the first page's section 0x09
//    describes the head sharing).
//  * A workgroup of four wavefronts owns one key range of one K/V head; the
//    wavefronts take every fourth 32-key tile of the range, each with its
//    own running statistics (the online softmax of the second page's
//    section 5), and merge their four results through LDS at the end.
//  * K goes straight from memory into registers in the A-operand layout of
//    v_mfma_f32_32x32x16_bf16 (16 bytes per lane); V goes into a per-
//    wavefront LDS double buffer with buffer_load ... lds (the range check
//    returns zeros past the last key) and is read back transposed with
//    ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T.  The loads for the
//    next tile are in flight while the current one is computed.
//
// Products are transposed as in the prefill kernel (fa_fwd_bf16.hip):
// S^T = K Q^T puts one query row per lane (lane % 32), and with the K rows
// fed in the order that swaps bits 2 and 3 of the key index, accumulator
// register i of lane half hf holds key 16*(i/8) + 8*hf + (i%8), which is
// where the B operand P^T of the next product expects it.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kRows = 32;      // packed query rows per workgroup
constexpr int kKeys = 32;      // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x32 product (D = A*B + C); lane l holds row/column l % 16 of A/B and
// the K slots of group l / 16, and rows 4*(l/16) .. +3 of column l % 16 of D.
__device__ __forceinline__ f32x4_t mfma16_bf16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Combine a value of this lane with the one of lane ^ 32 (v_permlane32_swap).
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

// V tile chunk permutation: the 4 rows x 4 chunks one phase of the transpose
// read touches land in 16 distinct bank groups.
template <int D> __device__ __forceinline__ int v_swz(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ void load_lds16(const void *base, int range, uint32_t off, lds_void_t *dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void vm_wait_all()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(kThreads, 2) decode_bf16_kernel(FwdParams p)
{
    constexpr int KSTEPS = D / 16;                  // K-steps of S^T = K Q^T
    constexpr int XB = D / 32;                      // 32-row blocks of O^T
    constexpr int CHUNKS = D / 8;                   // 16-byte chunks per row
    constexpr int ROW_BYTES = D * 2;
    constexpr int ROWS_PER_BLK = 1024 / ROW_BYTES;  // V rows per 1 KB direct load
    constexpr int VBLKS = kKeys * ROW_BYTES / 1024; // direct loads per V tile
    constexpr int TILE = kKeys * D;                 // elements of one V tile
    constexpr int HALF = D / 2;                     // floats per half row in the merge
    constexpr int HCH = HALF / 4;                   // 16-byte chunks per half row

    // Per-wavefront V double buffer (two objects, so the compiler sees that
    // the loads into one never alias the reads of the other).  After the
    // loop they hold the four wavefronts' unnormalised outputs for the merge,
    // columns [0, D/2) in Vs0 and [D/2, D) in Vs1 (fp32, exactly the size).
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[kWaves * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs1[kWaves * TILE];
    __shared__ float Mm[kWaves * kRows], Lm[kWaves * kRows], LBm[kWaves * kRows];

    // ---- workgroup -> (batch, K/V head, key range, row block)
    const int nrb = (p.Nq * p.group + kRows - 1) / kRows;
    int L = blockIdx.x;
    const int rb = L % nrb;
    L /= nrb;
    const int split = L % p.nsplit;
    L /= p.nsplit;
    const int hk = L % p.Hkv;
    const int b = L / p.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hf = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = p.off, g = p.group;
    const float c = p.c;

    // packed row of this lane: query row qi of query head hk*g + hh
    const int prow = rb * kRows + lq;
    const int qi = prow / g, hh = prow - (prow / g) * g;
    const bool row_ok = qi < Nq;
    const int h = hk * g + hh;
    // last key any valid row of this block can see, and the smallest such limit
    const int last_row = min(Nq - 1, (rb * kRows + kRows - 1) / g);
    const int first_row = (rb * kRows) / g;
    const int row_lim = CAUSAL ? min(qi + off, Nk - 1) : Nk - 1;

    // ---- key range of this workgroup, in 32-key tiles
    const int key_lo = split * p.split_keys;
    int key_hi = min(Nk, key_lo + p.split_keys);
    if (CAUSAL) key_hi = min(key_hi, last_row + off + 1);
    const int ntile = key_hi > key_lo ? (key_hi - key_lo + kKeys - 1) / kKeys : 0;
    const int my_n = ntile > wave ? (ntile - wave + kWaves - 1) / kWaves : 0;
    const int wave_lim = CAUSAL ? min(first_row + off, Nk - 1) : Nk - 1;   // keys <= this need no mask

    const int sK = p.Hkv * D;
    const uint16_t *kbase = (const uint16_t *)p.k + ((int64_t)b * Nk * p.Hkv + hk) * D;
    const uint16_t *vbase = (const uint16_t *)p.v + ((int64_t)b * Nk * p.Hkv + hk) * D;
    const int vrange = Nk * sK * 2;

    // ---- Q^T operand: lane (lq, hf) holds q[qi][h][16t + 8hf .. +7] for step t
    u32x4_t qreg[KSTEPS];
    if (row_ok && p.qmode != 2) {
        const u32x4_t *src = (const u32x4_t *)((const uint16_t *)p.q + (((int64_t)b * Nq + qi) * p.Hq + h) * D);
        const uint32_t flip = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            qreg[t] = src[2 * t + hf];
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[t][e] ^= flip;
        }
    } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qreg[t] = u32x4_t{0, 0, 0, 0};
    }

    // K row of the A operand for lane lq (bits 2 and 3 of the index swapped)
    const int krow = (lq & 0x13) | ((lq & 4) << 1) | ((lq & 8) >> 1);
    // V direct loads: lane l fills physical chunk l % CHUNKS of row l / CHUNKS
    const int ld_row = lane / CHUNKS, ld_pch = lane % CHUNKS;
    // transpose-read addressing (lane group tg = lane / 16, ts = lane % 16)
    const int tg = lane >> 4, ts = lane & 15;
    const int tr_row = 8 * (tg >> 1) + (ts >> 2);
    const int tr_chunk = 2 * (tg & 1) + ((ts & 3) >> 1);
    const int tr_byte = 8 * (ts & 1);

    auto tile_key0 = [&](int i) { return key_lo + (wave + i * kWaves) * kKeys; };

    // Start the loads of this wavefront's i-th tile: V into `vst`, K into kr.
    auto issue = [&](int i, uint16_t *vst, u32x4_t (&kr)[KSTEPS]) {
        const int key0 = tile_key0(i);
#pragma unroll
        for (int blk = 0; blk < VBLKS; ++blk) {
            const int row = blk * ROWS_PER_BLK + ld_row;
            const uint32_t off_b = (uint32_t)(key0 + row) * (uint32_t)(sK * 2) + ((ld_pch ^ v_swz<D>(row)) * 16);
            load_lds16(vbase, vrange, off_b, (lds_void_t *)&vst[wave * TILE + blk * 512]);
        }
        const int key = min(key0 + krow, Nk - 1);          // past the end: any valid row, masked below
        const u32x4_t *src = (const u32x4_t *)(kbase + (int64_t)key * sK);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) kr[t] = src[2 * t + hf];
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[XB];
    // The sum of the bf16 probabilities is taken on the matrix cores: one
    // 16x16x32 product per 16 keys with the P^T quad as B operand and a 0/1
    // selector as A, so that every accumulator register of lane l holds the
    // sum for its own query row l % 32 over both lane halves (rows 4r .. 4r+3
    // of the output take the K groups g = l / 16 with g % 2 == r % 2).  A
    // v_dot2 on the vector ALU would wait for the matrix pipeline while
    // another wavefront of the SIMD issues products.
    f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t sel_w = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x3f803f80u : 0u;
    const u32x4_t sum_sel = {sel_w, sel_w, sel_w, sel_w};
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[xb][i] = 0.f;

    auto compute = [&](int i, const uint16_t *vst, const u32x4_t (&kr)[KSTEPS]) {
        const int key0 = tile_key0(i);
        f32x16_t s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) s = mfma_bf16(kr[t], qreg[t], s);
        if (key0 + kKeys - 1 > wave_lim) {
            const int lim = row_lim - (key0 + 8 * hf);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (16 * (e >> 3) + (e & 7) > lim) s[e] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
        const float m_new = fmaxf(m_run, max_halves(mx) * c);
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
        m_run = m_new;
        u32x4_t pb[2];
        float rf = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * u + 2 * w2], c, -m_sub));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * u + 2 * w2 + 1], c, -m_sub));
                rf += e0 + e1;
                pb[u][w2] = pack_bf16(e0, e1);
            }
        l_run = l_run * alpha + rf;
        lacc *= alpha;
#pragma unroll
        for (int u = 0; u < 2; ++u) lacc = mfma16_bf16(sum_sel, pb[u], lacc);
        const char *vs = (const char *)&vst[wave * TILE];
#pragma unroll
        for (int xb = 0; xb < XB; ++xb) {
            oacc[xb] *= alpha;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4_t a;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int row = 16 * u + 4 * r + tr_row;
                    const int o_b = row * ROW_BYTES + (((4 * xb + tr_chunk) ^ v_swz<D>(row)) * 16) + tr_byte;
                    const i16x4_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + o_b));
                    const u32x2_t t2 = __builtin_bit_cast(u32x2_t, t4);
                    a[2 * r] = t2[0];
                    a[2 * r + 1] = t2[1];
                }
                oacc[xb] = mfma_bf16(a, pb[u], oacc[xb]);
            }
        }
    };

    // ---- main loop, two tiles per iteration so that both buffers are named statically
    u32x4_t kA[KSTEPS], kB[KSTEPS];
    if (my_n > 0) issue(0, Vs0, kA);
    for (int i = 0; i < my_n; i += 2) {
        vm_wait_all();                                   // tile i resident
        if (i + 1 < my_n) issue(i + 1, Vs1, kB);
        compute(i, Vs0, kA);
        if (i + 1 < my_n) {
            vm_wait_all();                               // tile i+1 resident
            if (i + 2 < my_n) issue(i + 2, Vs0, kA);
            compute(i + 1, Vs1, kB);
        }
    }

    // ---- merge the four wavefronts (m in base-2 units; O unnormalised)
    const float l_tot = sum_halves(l_run);
    const float lb_tot = lacc[0];
    __syncthreads();                                     // every V tile has been read
    if (hf == 0) {
        Mm[wave * kRows + lq] = m_run;
        Lm[wave * kRows + lq] = l_tot;
        LBm[wave * kRows + lq] = lb_tot;
    }
    // element (w, r, x) at half x / HALF, float (w*kRows + r)*HALF + 4*(chunk ^ (r % HCH)) + x % 4
#pragma unroll
    for (int xb = 0; xb < XB; ++xb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int x = xb * 32 + 8 * gi + 4 * hf;
            float *oh = (xb < XB / 2) ? (float *)Vs0 : (float *)Vs1;
            const int ch = ((x % HALF) / 4) ^ (lq % HCH);
            const f32x4_t w4 = {oacc[xb][4 * gi], oacc[xb][4 * gi + 1], oacc[xb][4 * gi + 2], oacc[xb][4 * gi + 3]};
            *(f32x4_t *)&oh[(wave * kRows + lq) * HALF + 4 * ch] = w4;
        }
    __syncthreads();

    constexpr int TPR = kThreads / kRows;   // threads per row
    constexpr int XPT = D / TPR;            // elements per thread
    const int r = tid / TPR, x0 = (tid % TPR) * XPT;
    const int pr = rb * kRows + r;
    const int rq = pr / g, rh = hk * g + (pr - (pr / g) * g);
    if (rq >= Nq) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, Mm[w * kRows + r]);
    float wgt[kWaves], Lt = 0.f, LBt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float mw = Mm[w * kRows + r];
        wgt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        Lt += wgt[w] * Lm[w * kRows + r];
        LBt += wgt[w] * LBm[w * kRows + r];
    }
    const bool empty = !(Lt > 0.f);
    const float inv = empty ? 0.f : 1.f / LBt;
    const float lse_row = empty ? -INFINITY : M * kLn2 + logf(Lt);
    const int64_t row = ((int64_t)split * p.B + b) * p.Hq + rh;   // split = 0 unless SPLIT
    const float *oh = x0 < HALF ? (const float *)Vs0 : (const float *)Vs1;
#pragma unroll
    for (int x = 0; x < XPT; x += 4) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const int ch = (((x0 + x) % HALF) / 4) ^ (r % HCH);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += wgt[w] * *(const f32x4_t *)&oh[(w * kRows + r) * HALF + 4 * ch];
        acc *= inv;
        if (SPLIT) {
            *(f32x4_t *)(p.o_part + (row * Nq + rq) * D + x0 + x) = acc;
        } else {
            const u32x2_t w2 = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
            *(u32x2_t *)((uint16_t *)p.o + (((int64_t)b * Nq + rq) * p.Hq + rh) * D + x0 + x) = w2;
        }
    }
    if (x0 == 0) (SPLIT ? p.lse_part : p.lse)[row * Nq + rq] = lse_row;
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_one(const FwdParams &p, hipStream_t stream)
{
    const int nrb = (p.Nq * p.group + kRows - 1) / kRows;
    const unsigned grid = (unsigned)p.B * (unsigned)p.Hkv * (unsigned)p.nsplit * (unsigned)nrb;
    hipLaunchKernelGGL((decode_bf16_kernel<D, CAUSAL, SPLIT>), dim3(grid), dim3(kThreads), 0, stream, p);
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

hipError_t launch_decode_bf16(const FwdParams &p, int d, hipStream_t stream)
{
    return d == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace fa
