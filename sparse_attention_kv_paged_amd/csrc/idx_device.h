// Device helpers shared by the score and top-k kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// Order-preserving map of a logit onto uint32: larger logit -> larger key.
// -0.0 and +0.0 map to one key (they are equal values); -inf and NaN map to
// 0, the "never selectable" key (masked columns are -inf).
__device__ __forceinline__ uint32_t order_key(float v) {
    if (!(v > -__builtin_inff())) return 0u;        // -inf or NaN
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(u);
}

// Inclusive prefix sum over the 256 threads of a workgroup (4 waves of 64).
// `sh` is 4 words of LDS.  Every thread of the workgroup must call it.
__device__ __forceinline__ uint32_t block_incl_scan256(uint32_t v, uint32_t *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) sh[wave] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int i = 0; i < wave; ++i) add += sh[i];
    __syncthreads();
    return v + add;
}

// Rank search over an LDS histogram of `nbins` (a multiple of 256) counts.
// FROM_TOP: find bin t with  count(bins > t) < need <= count(bins >= t);
// otherwise bin t with       count(bins < t) < need <= count(bins <= t).
// Writes t (or -1 when the total is below need) and the count strictly
// beyond t ("above" / "below") to res[0], res[1].  256 threads, all call.
template <bool FROM_TOP>
__device__ void find_rank_bin(const uint32_t *h, int nbins, uint32_t need,
                              int32_t *res, uint32_t *scan_sh) {
    const int tid = threadIdx.x;
    const int bpt = nbins >> 8;
    const int g = FROM_TOP ? (255 - tid) : tid;
    uint32_t local = 0;
    for (int i = 0; i < bpt; ++i) local += h[g * bpt + i];
    if (tid == 0) {
        res[0] = -1;
        res[1] = 0;
    }
    uint32_t incl = block_incl_scan256(local, scan_sh);
    uint32_t excl = incl - local;
    if (tid == 255 && incl < need) {
        res[0] = -1;
        res[1] = incl;
    }
    if (excl < need && need <= incl) {
        uint32_t c = excl;
        for (int i = 0; i < bpt; ++i) {
            int bin = FROM_TOP ? (g * bpt + bpt - 1 - i) : (g * bpt + i);
            uint32_t n = h[bin];
            if (c + n >= need) {
                res[0] = bin;
                res[1] = c;
                break;
            }
            c += n;
        }
    }
    __syncthreads();
}

}  // namespace idx
