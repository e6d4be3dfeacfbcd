// C ABI of libfa.so: argument validation, then one kernel launch.
// The operation, layouts, ownership and error behaviour are stated in
// include/fa.h.  Validation happens before any HIP call, so an invalid call
// enqueues nothing.
#include "fa.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int validate_and_fill(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                      size_t elem, fa::FwdParams &p)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEADS;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    // 32-bit byte offsets inside one batch entry (also for the up to 255 rows
    // past N that the kernels' range-checked loads may address), 32-bit grid
    const int64_t hmax = Hq > Hkv ? Hq : Hkv;
    if (((int64_t)N + 256) * hmax * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;
    const int64_t ntiles = ((int64_t)N + fa::kBlockM - 1) / fa::kBlockM;
    if ((int64_t)B * Hq * ntiles >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    const size_t nq = (size_t)B * N * Hq * d * elem;
    const size_t nk = (size_t)B * N * Hkv * d * elem;
    const size_t nl = (size_t)B * Hq * N * sizeof(float);
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nk) || overlaps(o, nq, v, nk) ||
        overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
        overlaps(o, nq, lse, nl))
        return FA_ERR_ALIAS;

    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N;
    p.group = Hq / Hkv;
    p.ntiles = (int)ntiles;
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

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 2, p);
    if (st != FA_OK) return st;
    return fa::launch_fwd_bf16(p, d, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, void *stream)
{
    fa::FwdParams p;
    const int st = validate_and_fill(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 4, p);
    if (st != FA_OK) return st;
    return fa::launch_fwd_f32(p, d, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char *fa_strerror(int status)
{
    switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, Hq, Hkv and N must be >= 1 and within the size limits";
    case FA_ERR_HEADS: return "Hq must be a multiple of Hkv";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite (and |scale|*log2(e) representable)";
    case FA_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case FA_ERR_LAUNCH: return "the HIP runtime reported an error for the kernel launch";
    default: return "unknown fa_status";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
