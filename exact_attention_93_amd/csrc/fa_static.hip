// fa_fwd_splitkv_static: the split forward for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its per-range partial results live in one file-scope device
// array, `scratch`, instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  Host code never uses the array's name as
// an address (in host code it names a host-side stand-in): the device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and only that pointer reaches the kernels.  Every call on one GPU
// shares that GPU's array and leaves its contents behind; the split kernels
// write every partial they later read, so nothing needs clearing.  Calls that
// overlap in time on one GPU race on the array: enqueue them on one stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)FA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// The device address of `scratch` on the current device, or NULL.
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    __atomic_store_n(&g_scratch[dev], p, __ATOMIC_RELEASE);
    return p;
}

}  // namespace

extern "C" int fa_fwd_splitkv_static(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                                     int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                                     int num_splits, void *stream)
{
    fa::FwdParams p;
    size_t need = 0;
    const int st = fa::splitkv_prepare(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, p, need);
    if (st != FA_OK) return st;
    if (need > kScratchBytes) return FA_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_address();
        if (!ws) return FA_ERR_LAUNCH;
    }
    return fa::splitkv_run(p, d, ws, (hipStream_t)stream);
}
