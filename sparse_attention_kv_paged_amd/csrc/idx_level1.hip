// Level-1 resident-set selection for gfx950: the page pass between the
// per-layer scoring (score kernel, sigmoid output) and the top-KMAX page
// selection (segment top-k kernel) ("FlashMemory-DeepSeek-V4" README,
// sections "Two-level recall algorithm" and "Joint checkpoint + ensemble";
// KMAX pages of 64 entries per request, section "Quick start").
//
// A wave takes four consecutive 64-entry pages: lane l reads entries
// 4l .. 4l + 3 of the 256 (one 16-byte load per layer), ensembles them (max,
// or the binary32 sum in layer order divided by L) and counts those at or
// above the threshold; a DPP row (16 lanes) covers one page, so four row
// rotations sum the page's density.  The page's key for the selection orders
// pages by (forced, density, lower page first) and is exact in binary32:
//     forced (sink or recent page)       (kMaxDensity + 1) * 2^17 + (2^17 - 1 - p)
//     density d > 0                      d * 2^17 + (2^17 - 1 - p)
//     otherwise (or past the history)    -inf
// so that every key of a row is distinct and the top-k's value-linear
// histogram separates them (a +inf or integer-only key would put whole tie
// groups in one bin).  Rows of more than 2^17 pages use keys d and +inf
// instead, which select the same pages through the top-k's own tie rule.
#include <hip/hip_runtime.h>

#include "../../include/idx.h"
#include "idx_internal.h"
#include "idx_level1.h"

namespace idx {
namespace {

constexpr int kPageWaves = 4;
constexpr int kPagesPerWave = 4;
constexpr int kPageBits = 17;

// The value of the lane N places further along this lane's 16-lane DPP row.
template <int N>
__device__ __forceinline__ int row_ror(int x) {
    return __builtin_amdgcn_update_dpp(0, x, 0x120 + N, 0xF, 0xF, false);
}

__global__ __launch_bounds__(64 * kPageWaves) void page_kernel(PageArgs a) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x % 64;
    const int p0 = (blockIdx.x * kPageWaves + threadIdx.x / 64) * kPagesPerWave;
    if (p0 >= a.n_pages) return;                      // uniform per wave
    const int hist = max(0, min(a.limits[b], a.n_cols));
    const int P = (hist + kBlock - 1) / kBlock;
    const int p = p0 + lane / 16;                      // this lane's page
    const int e0 = p0 * kBlock + 4 * lane;             // its first entry
    int count = 0;
    if (e0 < hist) {
        const float *row = a.scores + (int64_t)b * a.ld + e0;
        float s[4];
        // the four entries are in bounds of the row stride (ld is a multiple
        // of 64); entries past hist are not counted
        float4 x = *reinterpret_cast<const float4 *>(row);
        s[0] = x.x; s[1] = x.y; s[2] = x.z; s[3] = x.w;
        for (int l = 1; l < a.L; ++l) {
            x = *reinterpret_cast<const float4 *>(row + (int64_t)l * a.layer_stride);
            const float y[4] = {x.x, x.y, x.z, x.w};
            if (a.ensemble == IDX_ENSEMBLE_MAX) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = y[i] > s[i] ? y[i] : s[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] += y[i];
            }
        }
        if (a.ensemble == IDX_ENSEMBLE_MEAN) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = s[i] / (float)a.L;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) count += (e0 + i < hist && s[i] >= a.threshold) ? 1 : 0;
    }
    count += row_ror<8>(count);
    count += row_ror<4>(count);
    count += row_ror<2>(count);
    count += row_ror<1>(count);
    if (lane % 16 == 0 && p < a.n_pages) {
        const bool forced = p < P && (p < a.n_sink || p >= P - a.n_recent);
        float key = -__builtin_inff();
        if (a.n_pages <= (1 << kPageBits)) {
            const int tie = (1 << kPageBits) - 1 - p;
            if (forced) key = (float)((kBlock + 1) * (1 << kPageBits) + tie);
            else if (p < P && count > 0) key = (float)(count * (1 << kPageBits) + tie);
        } else {
            if (forced) key = __builtin_inff();
            else if (p < P && count > 0) key = (float)count;
        }
        a.page_keys[(int64_t)b * a.ldp + p] = key;
    }
}

// The same page keys from the score launch's selection bits (max ensemble:
// an entry is selected iff some layer's score reaches the threshold, so the
// page's selected entries are the OR of the layers' words): one thread per
// page, entries at or past the row's history masked off.
__global__ __launch_bounds__(256) void page_bits_kernel(PageArgs a) {
    const int b = blockIdx.y;
    const int p = blockIdx.x * 256 + (int)threadIdx.x;
    if (p >= a.n_pages) return;
    const int hist = max(0, min(a.limits[b], a.n_cols));
    const int P = (hist + kBlock - 1) / kBlock;
    uint64_t m = 0;
    for (int l = 0; l < a.L; ++l) {
        const uint32_t *row = a.bits + ((int64_t)l * a.B + b) * a.bits_ld;
        m |= (uint64_t)row[2 * p] | ((uint64_t)row[2 * p + 1] << 32);
    }
    const int valid = max(0, min(hist - p * kBlock, kBlock));
    m = valid == 0 ? 0 : valid == kBlock ? m : m & ((1ull << valid) - 1);
    const int count = __popcll(m);
    const bool forced = p < P && (p < a.n_sink || p >= P - a.n_recent);
    float key = -__builtin_inff();
    if (a.n_pages <= (1 << kPageBits)) {
        const int tie = (1 << kPageBits) - 1 - p;
        if (forced) key = (float)((kBlock + 1) * (1 << kPageBits) + tie);
        else if (p < P && count > 0) key = (float)(count * (1 << kPageBits) + tie);
    } else {
        if (forced) key = __builtin_inff();
        else if (p < P && count > 0) key = (float)count;
    }
    a.page_keys[(int64_t)b * a.ldp + p] = key;
}

}  // namespace

hipError_t launch_pages(const PageArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.n_pages <= 0) return hipSuccess;
    if (a.bits) {
        if (a.ensemble != IDX_ENSEMBLE_MAX || a.bits_ld < 2 * (int64_t)a.n_pages) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((a.n_pages + 255) / 256), (unsigned)a.B);
        hipLaunchKernelGGL(page_bits_kernel, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const int per_group = kPageWaves * kPagesPerWave;
    const dim3 grid((unsigned)((a.n_pages + per_group - 1) / per_group), (unsigned)a.B);
    hipLaunchKernelGGL(page_kernel, grid, dim3(64 * kPageWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace idx
