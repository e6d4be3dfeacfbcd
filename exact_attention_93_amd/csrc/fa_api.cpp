// C ABI of libfa.so: argument validation, then the kernel launches.
// The operation, layouts, ownership and error behaviour are stated in
// include/fa.h.  Validation happens before any HIP call, so an invalid call
// enqueues nothing.
#include "fa.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace {

constexpr int kVersion = 200;  // 0.2.0
constexpr int kMaxSplits = 256;

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Key range of one split: a multiple of the split quantum, and the number of
// ranges that are actually used (never more than requested, none empty).
void split_shape(int Nk, int num_splits, int &split_keys, int &nsplit)
{
    const int64_t quanta = cdiv(Nk, fa::kSplitQuantum);
    const int64_t per = cdiv(quanta, num_splits);
    split_keys = (int)(per * fa::kSplitQuantum);
    nsplit = (int)cdiv(quanta, per);
}

int heuristic_splits(int B, int Hq, int Hkv, int Nq, int Nk)
{
    // Aim at one full round of workgroups over the 256 compute units: the
    // decoding kernel (one workgroup per K/V head and packed row block) gets
    // ranges of at least 1024 keys; the prefill kernel (one workgroup per
    // query head and 256 query rows, one per compute unit) takes the range
    // count with the fewest rounds per unit of work, ranges of at least 256
    // keys.
    constexpr int kCUs = 256;
    const int group = Hq / Hkv;
    if (fa::use_decode(Nq, group)) {
        const int64_t units = (int64_t)B * Hkv * cdiv((int64_t)Nq * group, fa::kDecodeRowBlock);
        int64_t s = cdiv(kCUs, units);
        const int64_t max_by_len = cdiv(Nk, 1024);
        if (s > max_by_len) s = max_by_len;
        if (s > kMaxSplits) s = kMaxSplits;
        return s < 1 ? 1 : (int)s;
    }
    const int64_t units = (int64_t)B * Hq * cdiv(Nq, 256);
    if (units >= kCUs) return 1;
    int64_t max_s = cdiv(Nk, 4 * fa::kSplitQuantum);
    if (max_s > kMaxSplits) max_s = kMaxSplits;
    int best = 1;
    double best_cost = 1.0 * cdiv(units, kCUs);
    for (int s = 2; s <= max_s; ++s) {
        const double cost = (double)cdiv(units * s, kCUs) / s * (1.0 + 0.02 * s);
        if (cost < best_cost) { best_cost = cost; best = s; }
    }
    return best;
}

size_t workspace_bytes_for(int B, int Hq, int Nq, int d, int nsplit)
{
    return (size_t)nsplit * B * Hq * Nq * (size_t)(d + 1) * sizeof(float);
}

int validate_and_fill(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int num_splits, void *ws, size_t ws_bytes, size_t elem, fa::FwdParams &p,
                      size_t out_elem = 0, bool allow_d256 = false, bool defer_ws = false)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEADS;
    if (d != 64 && d != 128 && !(allow_d256 && d == 256)) return FA_ERR_HEADDIM;
    if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
    if (num_splits == 0) num_splits = heuristic_splits(B, Hq, Hkv, Nq, Nk);
    int split_keys, nsplit;
    split_shape(Nk, num_splits, split_keys, nsplit);
    // 32-bit element offsets inside one batch entry (also for the up to 255
    // rows past the end that the kernels' range-checked loads may address),
    // 32-bit grids
    if (((int64_t)Nq + 256) * Hq * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    if (((int64_t)Nk + 256) * Hkv * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    const int64_t ntiles = cdiv(Nq, fa::kBlockM);
    if ((int64_t)B * Hq * ntiles * nsplit >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    if ((int64_t)B * Hkv * cdiv((int64_t)Nq * (Hq / Hkv), fa::kDecodeRowBlock) * nsplit >= ((int64_t)1 << 31))
        return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    if (out_elem == 0) out_elem = elem;
    const size_t nq = (size_t)B * Nq * Hq * d * elem;
    const size_t no = (size_t)B * Nq * Hq * d * out_elem;
    const size_t nk = (size_t)B * Nk * Hkv * d * elem;
    const size_t nl = (size_t)B * Hq * Nq * sizeof(float);
    if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nk) ||
        overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
        overlaps(o, no, lse, nl))
        return FA_ERR_ALIAS;
    p.o_part = nullptr;
    p.lse_part = nullptr;
    p.q_descale = p.k_descale = p.v_descale = nullptr;
    p.q_exp = p.k_exp = p.v_exp = nullptr;
    p.block_mask = nullptr;
    p.mask_nqb = p.mask_nkb = 0;
    if (nsplit > 1 && !defer_ws) {
        const size_t need = workspace_bytes_for(B, Hq, Nq, d, nsplit);
        if (!ws || ws_bytes < need || ((uintptr_t)ws & 15)) return FA_ERR_WORKSPACE;
        if (overlaps(ws, need, q, nq) || overlaps(ws, need, k, nk) || overlaps(ws, need, v, nk) ||
            overlaps(ws, need, o, no) || overlaps(ws, need, lse, nl))
            return FA_ERR_ALIAS;
        p.o_part = (float *)ws;
        p.lse_part = (float *)ws + (size_t)nsplit * B * Hq * Nq * d;
    }

    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
    p.off = Nk - Nq;
    p.group = Hq / Hkv;
    p.ntiles = (int)ntiles;
    p.nsplit = nsplit;
    p.split_keys = split_keys;
    p.causal = causal ? 1 : 0;
    p.xcd_groups = ((B * Hkv) % 8 == 0) ? 1 : 0;
    // The kernels take a positive base-2 scale.  A negative scale is the same
    // as negating q (exact for bf16 and fp32); a zero scale makes every score
    // zero, which the kernels realise by zeroing q.
    if (scale > 0.f) {
        p.qmode = 0;
        p.c = (float)((double)scale * 1.4426950408889634);
    } else if (scale < 0.f) {
        p.qmode = 1;
        p.c = (float)(-(double)scale * 1.4426950408889634);
    } else {
        p.qmode = 2;
        p.c = 1.f;
    }
    if (!(p.c >= FLT_MIN) || !isfinite(p.c)) return FA_ERR_SCALE;  // |scale|*log2(e) not a normal float
    return FA_OK;
}

// HIP keeps the error of the last failing runtime call until it is read, and a
// successful launch does not reset it.  Cleared right before this library's
// launches, so that the check after each launch sees only that launch (an
// earlier failure elsewhere in the process was returned to its own caller).
void clear_stale_error() { (void)hipGetLastError(); }

int run(const fa::FwdParams &p, int d, bool bf16, hipStream_t stream)
{
    clear_stale_error();
    hipError_t e;
    if (!bf16) e = fa::launch_fwd_f32(p, d, stream);
    else if (d <= 128 && !p.block_mask && fa::use_decode(p.Nq, p.group)) e = fa::launch_decode_bf16(p, d, stream);
    else e = fa::launch_fwd_bf16(p, d, stream);
    if (e != hipSuccess) return FA_ERR_LAUNCH;
    if (p.nsplit > 1 && fa::launch_combine(p, d, bf16 ? 1 : 0, stream) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
}

}  // namespace

namespace fa {

int splitkv_prepare(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                    int Nq, int Nk, int d, float scale, int causal, int num_splits, FwdParams &p,
                    size_t &ws_need)
{
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits,
                                     nullptr, 0, 2, p, 0, true, true);
    if (st != FA_OK) return st;
    ws_need = p.nsplit > 1 ? workspace_bytes_for(B, Hq, Nq, d, p.nsplit) : 0;
    return FA_OK;
}

int splitkv_run(FwdParams &p, int d, void *ws, hipStream_t stream)
{
    if (p.nsplit > 1) {
        p.o_part = (float *)ws;
        p.lse_part = (float *)ws + (size_t)p.nsplit * p.B * p.Hq * p.Nq * (size_t)d;
    }
    return run(p, d, true, stream);
}

}  // namespace fa

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, causal, 1,
                                     nullptr, 0, 2, p, 0, true);
    return st != FA_OK ? st : run(p, d, true, (hipStream_t)stream);
}

int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, causal, 1,
                                     nullptr, 0, 4, p);
    return st != FA_OK ? st : run(p, d, false, (hipStream_t)stream);
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int num_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                                     num_splits, workspace, workspace_bytes, 2, p, 0, true);
    return st != FA_OK ? st : run(p, d, true, (hipStream_t)stream);
}

int fa_fwd_splitkv_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       int num_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                                     num_splits, workspace, workspace_bytes, 4, p);
    return st != FA_OK ? st : run(p, d, false, (hipStream_t)stream);
}

int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv != 0) return -FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return -FA_ERR_HEADDIM;
    if (num_splits < 0 || num_splits > kMaxSplits) return -FA_ERR_SPLITS;
    if (num_splits == 0) num_splits = heuristic_splits(B, Hq, Hkv, Nq, Nk);
    int split_keys, nsplit;
    split_shape(Nk, num_splits, split_keys, nsplit);
    return nsplit;
}

size_t fa_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits)
{
    const int nsplit = fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits);
    if (nsplit <= 1) return 0;
    return workspace_bytes_for(B, Hq, Nq, d, nsplit);
}

int fa_fwd_blocksparse(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       const unsigned char *block_mask, void *stream)
{
    if (!block_mask) return FA_ERR_NULL;
    if (N > 65536) return (!q || !k || !v || !o || !lse) ? FA_ERR_NULL : FA_ERR_SHAPE;
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, causal, 1,
                                     nullptr, 0, 2, p, 0, true);
    if (st != FA_OK) return st;
    p.block_mask = block_mask;
    p.mask_nqb = (int)cdiv(N, 128);
    p.mask_nkb = (int)cdiv(N, 64);
    return run(p, d, true, (hipStream_t)stream);
}

int fa_fwd_fp8(const void *q, const void *k, const void *v, const float *q_descale,
               const float *k_descale, const float *v_descale, void *o, float *lse, int B, int Hq,
               int Hkv, int N, int d, float scale, int causal, void *stream)
{
    if (!q_descale || !k_descale || !v_descale) return FA_ERR_NULL;
    if (d != 128) return (!q || !k || !v || !o || !lse) ? FA_ERR_NULL : FA_ERR_HEADDIM;
    if (((uintptr_t)q_descale | (uintptr_t)k_descale | (uintptr_t)v_descale) & 3) return FA_ERR_ALIGN;
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, causal, 1,
                                     nullptr, 0, 1, p, 2);
    if (st != FA_OK) return st;
    p.q_descale = q_descale;
    p.k_descale = k_descale;
    p.v_descale = v_descale;
    clear_stale_error();
    return fa::launch_fwd_fp8(p, d, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_fp8_block(const void *q, const void *k, const void *v, const signed char *q_exp,
                     const signed char *k_exp, const signed char *v_exp, void *o, float *lse, int B, int Hq,
                     int Hkv, int N, int d, float scale, int causal, void *stream)
{
    if (!q_exp || !k_exp || !v_exp) return FA_ERR_NULL;
    if (d != 128) return (!q || !k || !v || !o || !lse) ? FA_ERR_NULL : FA_ERR_HEADDIM;
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, causal, 1,
                                     nullptr, 0, 1, p, 2);
    if (st != FA_OK) return st;
    // the exponent arrays must not overlap the outputs
    const size_t nb = (size_t)cdiv(N, fa::kQuantBlock);
    const size_t no = (size_t)B * N * Hq * d * 2, nl = (size_t)B * Hq * N * sizeof(float);
    const void *ex[3] = {q_exp, k_exp, v_exp};
    const size_t exn[3] = {(size_t)B * Hq * nb, (size_t)B * Hkv * nb, (size_t)B * Hkv * nb};
    for (int i = 0; i < 3; ++i)
        if (overlaps(o, no, ex[i], exn[i]) || overlaps(lse, nl, ex[i], exn[i])) return FA_ERR_ALIAS;
    p.q_exp = (const int8_t *)q_exp;
    p.k_exp = (const int8_t *)k_exp;
    p.v_exp = (const int8_t *)v_exp;
    clear_stale_error();
    return fa::launch_fwd_fp8(p, d, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_quantize_fp8(const void *x, void *codes, signed char *exps, int B, int N, int H, int d,
                    const signed char *signs, void *stream)
{
    if (!x || !codes || !exps) return FA_ERR_NULL;
    if (B < 1 || N < 1 || H < 1) return FA_ERR_SHAPE;
    if (d != 128) return FA_ERR_HEADDIM;
    if (((int64_t)N + fa::kQuantBlock) * H * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    const int64_t nb = cdiv(N, fa::kQuantBlock);
    if ((int64_t)B * H * nb >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    if (((uintptr_t)x & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)signs & 7)) return FA_ERR_ALIGN;
    const size_t nx = (size_t)B * N * H * d * 2, nc = (size_t)B * N * H * d, ne = (size_t)B * H * nb;
    if (overlaps(codes, nc, x, nx) || overlaps(exps, ne, x, nx) || overlaps(exps, ne, codes, nc) ||
        (signs && (overlaps(signs, d, codes, nc) || overlaps(signs, d, exps, ne))))
        return FA_ERR_ALIAS;
    fa::QuantParams p;
    p.x = x;
    p.codes = codes;
    p.exps = (int8_t *)exps;
    p.signs = (const int8_t *)signs;
    p.B = B; p.N = N; p.H = H;
    clear_stale_error();
    return fa::launch_quant_fp8(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq)
{
    if (B < 1 || Hq < 1 || Nq < 1) return 0;
    return 2 * (size_t)B * Hq * Nq * sizeof(float);   // delta, then lse in base 2
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Nq, int Nk,
           int d, float scale, int causal, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEADS;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (((int64_t)Nq + 256) * Hq * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    if (((int64_t)Nk + 256) * Hkv * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    if ((int64_t)B * Hq * cdiv(Nq, 128) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    if ((int64_t)B * Hkv * cdiv(Nk, 128) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15)
        return FA_ERR_ALIGN;
    if (((uintptr_t)lse | (uintptr_t)workspace) & 3) return FA_ERR_ALIGN;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    const size_t need = fa_bwd_workspace_size(B, Hq, Nq);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    const size_t nq = (size_t)B * Nq * Hq * d * 2, nk = (size_t)B * Nk * Hkv * d * 2;
    const size_t nl = (size_t)B * Hq * Nq * sizeof(float);
    const void *ins[6] = {q, k, v, o, dout, lse};
    const size_t insz[6] = {nq, nk, nk, nq, nq, nl};
    void *outs[4] = {dq, dk, dv, workspace};
    const size_t outsz[4] = {nq, nk, nk, need};
    for (int a = 0; a < 4; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[a], outsz[a], ins[i], insz[i])) return FA_ERR_ALIAS;
        for (int c2 = a + 1; c2 < 4; ++c2)
            if (overlaps(outs[a], outsz[a], outs[c2], outsz[c2])) return FA_ERR_ALIAS;
    }

    fa::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.delta = (float *)workspace;
    p.lse2 = (float *)workspace + (size_t)B * Hq * Nq;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
    p.off = Nk - Nq;
    p.group = Hq / Hkv;
    p.causal = causal ? 1 : 0;
    p.xcd_groups = ((B * Hkv) % 8 == 0) ? 1 : 0;
    p.scale = scale;
    if (scale > 0.f) {
        p.qmode = 0;
        p.c = (float)((double)scale * 1.4426950408889634);
    } else if (scale < 0.f) {
        p.qmode = 1;
        p.c = (float)(-(double)scale * 1.4426950408889634);
    } else {
        p.qmode = 2;
        p.c = 1.f;
    }
    if (!(p.c >= FLT_MIN) || !isfinite(p.c)) return FA_ERR_SCALE;
    clear_stale_error();
    return fa::launch_bwd_bf16(p, d, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char *fa_strerror(int status)
{
    switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, Hq, Hkv and the sequence lengths must be >= 1 and within the size limits";
    case FA_ERR_HEADS: return "Hq must be a multiple of Hkv";
    case FA_ERR_HEADDIM: return "unsupported head dimension (bf16 forward: 64, 128, 256; fp32 forward: 64, 128; backward: 64, 128; fp8: 128)";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite (and |scale|*log2(e) representable)";
    case FA_ERR_ALIAS: return "an output or the workspace overlaps an input or another output";
    case FA_ERR_LAUNCH: return "the HIP runtime reported an error for the kernel launch";
    case FA_ERR_SPLITS: return "num_splits must be in 0..256";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the size function returns (split forward: also 16-byte aligned)";
    case FA_ERR_SCRATCH: return "the split forward needs more scratch memory than the library's static array holds";
    default: return "unknown fa_status";
    }
}

int fa_version(void) { return kVersion; }

int fa_lds_stages(void)
{
    const int n = fa::fwd_bf16_lds_stages();
    return (n == fa::fwd_fp8_lds_stages() && n == fa::fwd_f32_lds_stages() && n == fa::bwd_lds_stages()) ? n : 0;
}

}  // extern "C"
