// Internal interface between the C-ABI layer (fa_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Smallest number of query rows any kernel gives one workgroup (bounds the grid size).
constexpr int kBlockM = 128;

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, N;
    int group;       // Hq / Hkv: query heads sharing one key/value head
    int ntiles;      // query tiles per (batch, head); set by each kernel's launcher
    int causal;
    int xcd_groups;  // 1 when B*Hkv is a multiple of 8 (one XCD per head group)
    int qmode;       // 0: q as given; 1: q negated (scale < 0); 2: q zeroed (scale == 0)
    float c;         // |scale| * log2(e) (positive), or 1 when scale == 0
};

hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams &p, int d, hipStream_t stream);

// Workgroup index -> (batch, query head, query tile).
//
// Workgroups are dealt to the 8 XCDs round-robin by index, so index L runs
// on XCD L % 8.  When B*Hkv is a multiple of 8, XCD x is given every query
// tile of the key/value head groups g with g % 8 == x (all query heads that
// share a K/V head included), so the K/V of a head is fetched into one XCD's
// L2 only.  Within an XCD, causal tiles go heaviest first (the last query
// tile sees the most keys), which keeps the tail of the launch short.
__device__ __forceinline__ void decode_tile(const FwdParams &p, int &b, int &h, int &tile)
{
    const int L = blockIdx.x;
    int t;
    if (p.xcd_groups) {
        const int xcd = L & 7, s = L >> 3;
        const int heads_here = (p.B * p.Hkv >> 3) * p.group;
        t = s / heads_here;
        const int r = s - t * heads_here;
        const int lg = r / p.group, qh = r - lg * p.group;
        const int g = lg * 8 + xcd;
        b = g / p.Hkv;
        h = (g - b * p.Hkv) * p.group + qh;
    } else {
        const int per = p.B * p.Hq;
        t = L / per;
        const int r = L - t * per;
        b = r / p.Hq;
        h = r - b * p.Hq;
    }
    tile = p.causal ? (p.ntiles - 1 - t) : t;
}

}  // namespace fa
